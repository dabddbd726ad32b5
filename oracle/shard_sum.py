"""Oracle for the all-reduce that ends each tensor-parallel block.

The ranks' partials Z_i are added to give Z [Megatron-LM：张量并行与大规模训练,
§2.1 MLP 层的张量并行, row parallelism: Z = Z_1 + ... + Z_N; m.youleyou.com/wenzhang/
3143730, 二、MLP层 §2.1, g's forward adds Z_1 and Z_2]. On one GPU the N partials
are summed in place of the exchange.

The pages only say the partials are added. Reading: a fixed order
((P_0 + P_1) + P_2) + ... in float32, which makes the result unique and
reproducible; the float64 sum is the exact reference.
"""
import numpy as np

from .bf16 import bf16_bits_to_f64, f64_to_bf16_bits


def shard_sum_f64(parts):
    """Sum of the partials in float64."""
    acc = np.zeros(np.shape(parts[0]), np.float64)
    for p in parts:
        acc = acc + np.asarray(p, np.float64)
    return acc


def shard_sum_f32_ordered(parts):
    """float32 sum in the fixed order i = 0 .. N-1 (each add is one IEEE
    float32 round-to-nearest-even operation)."""
    acc = np.asarray(parts[0], np.float32).copy()
    for p in parts[1:]:
        acc = (acc + np.asarray(p, np.float32)).astype(np.float32)
    return acc


def shard_sum_bf16_ordered(parts_bits):
    """bfloat16 partials: widened exactly, summed in float32 in order, and the
    float32 result rounded once to bfloat16 (nearest even). Returns bit patterns."""
    acc = bf16_bits_to_f64(parts_bits[0]).astype(np.float32)
    for p in parts_bits[1:]:
        acc = (acc + bf16_bits_to_f64(p).astype(np.float32)).astype(np.float32)
    return f64_to_bf16_bits(acc.astype(np.float64))
