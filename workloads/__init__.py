"""Seeded synthetic workloads shared by the CPU oracle's tests, the GPU parity
tests and the benchmark.

This package only draws random numbers and slices them into per-rank shards.
It holds none of the method's arithmetic: no GEMM, activation, softmax, sum or
gather lives here. Rounding of the drawn fp32 samples to bfloat16 storage is
done by torch's CPU conversion (round-to-nearest-even), a library routine, so
that neither the oracle nor the HIP path supplies its own inputs.
"""
from .gen import (  # noqa: F401
    CONFIGS,
    bf16_bits,
    bf16_bits_to_f32,
    draw_normal_f32,
    mlp_inputs,
    attn_inputs,
    embed_inputs,
    ce_inputs,
    sp_inputs,
    shard_sum_inputs,
    shard_cols,
    shard_rows,
)
