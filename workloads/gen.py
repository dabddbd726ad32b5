"""Seeded input generators for the five workloads of the rank-shard path.

Shapes follow the per-rank shard of a Megatron-style Transformer layer
[Megatron-LM：张量并行与大规模训练, §2.1 MLP 层的张量并行 and §2.2 Self-Attention
的张量并行]: X is [b*s, h] and identical on every rank; the MLP weight A is split by
columns into A_i [h, 4h/N] and B by rows into B_i [4h/N, h]; attention heads are
split into contiguous blocks of H/N heads; the word-embedding table is split by
rows into contiguous vocabulary ranges [lo, hi) [m.youleyou.com/wenzhang/3143730,
四、Embedding层 §4.1]. The GPT-3 175B sizes (h = 12288, 96 heads, context 2048)
come from the same page's table [Megatron-LM：张量并行与大规模训练, §5.6].

Recipe: ``np.random.default_rng(seed)``; tensors are drawn in the listed order as
float32 standard normals times sigma (computed in float32); bfloat16 tensors are
then rounded to nearest-even by torch on the CPU and handed over as uint16 bit
patterns. Token ids are uniform int32 in [0, v).
"""
from __future__ import annotations

import numpy as np
import torch

# name -> shapes and distributions of each workload. "seed" is the generator seed.
CONFIGS = {
    "tiny_mlp_fp32": dict(name="tiny_mlp_fp32", b=1, s=8, h=64, f_full=256, N=2, dtype="f32",
            sigma_x=1.0, sigma_w=0.02, seed=1001),
    "small_mlp_bf16": dict(name="small_mlp_bf16", b=1, s=32, h=1024, f_full=4096, N=2, dtype="bf16",
            sigma_x=1.0, sigma_w=0.02, sigma_dz=1.0, seed=1002),
    "gpt3_mlp_rank_shard": dict(name="gpt3_mlp_rank_shard", b=1, s=2048, h=12288, f=6144, N=8, dtype="bf16",
            sigma_x=1.0, sigma_w=0.006, sigma_dz=1.0, n_partials=8, sigma_p=1.0, seed=1003),
    "gpt3_attn_rank_shard": dict(name="gpt3_attn_rank_shard", b=1, s=2048, h=12288, n_heads=96, N=8,
            d_head=128, dtype="bf16", sigma_x=1.0, sigma_w=0.006, seed=1004),
    "vocab_parallel_embed": dict(name="vocab_parallel_embed", v=50304, N=8, h=12288, b=8, s=2048,
            dtype="bf16", sigma_w=0.02, seed=1005),
    # PaLM 540B rank shard (h = 18432, 48 heads, context 4096, TP = 8, f = 4h/8)
    # [Megatron-LM：张量并行与大规模训练, §5.7]: a second MLP shape and the attention
    # shard of 6 local heads of 18432 / 48 = 384.
    "palm_mlp_rank_shard": dict(name="palm_mlp_rank_shard", b=1, s=4096, h=18432, f=9216, N=8, dtype="bf16",
            sigma_x=1.0, sigma_w=0.005, sigma_dz=1.0, seed=1006),
    "palm_attn_rank_shard": dict(name="palm_attn_rank_shard", b=1, s=4096, h=18432, n_heads=48, N=8,
            d_head=384, dtype="bf16", sigma_x=1.0, sigma_w=0.005, seed=1009),
    # Vocabulary-parallel output layer + cross-entropy over the GPT-3 vocabulary
    # (padded to 50304 = 8 * 6288), one sequence of 2048 tokens.
    "vocab_parallel_ce": dict(name="vocab_parallel_ce", v=50304, N=8, h=12288, b=1, s=2048, dtype="bf16",
            sigma_h=1.0, sigma_w=0.02, seed=1007),
    # Sequence-parallel MLP block at the GPT-3 shard: LayerNorm on s/N rows per rank,
    # all-gather, reduce-scatter of 8 fp32 partials fused with dropout and residual.
    "gpt3_sp_mlp_block": dict(name="gpt3_sp_mlp_block", s=2048, h=12288, f=6144, N=8, sigma_r=1.0, sigma_g=0.1,
            sigma_b=0.1, keep_prob=0.9, sigma_p=1.0, seed=1008),
}


def draw_normal_f32(rng: np.random.Generator, shape, sigma: float) -> np.ndarray:
    """float32 N(0, sigma^2) samples (sigma is the standard deviation)."""
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if sigma != 1.0:
        x *= np.float32(sigma)
    return x


def bf16_bits(x32: np.ndarray) -> np.ndarray:
    """Round float32 samples to bfloat16 (torch CPU, nearest-even); return uint16 bits."""
    t = torch.from_numpy(np.ascontiguousarray(x32, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32 (a bit shift)."""
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32)


def _store(x32: np.ndarray, dtype: str) -> np.ndarray:
    return x32 if dtype == "f32" else bf16_bits(x32)


def shard_cols(W: np.ndarray, N: int, i: int) -> np.ndarray:
    """Columns [i*n/N, (i+1)*n/N) of W (column-parallel split)."""
    n = W.shape[1]
    assert n % N == 0
    w = n // N
    return np.ascontiguousarray(W[:, i * w:(i + 1) * w])


def shard_rows(W: np.ndarray, N: int, i: int) -> np.ndarray:
    """Rows [i*m/N, (i+1)*m/N) of W (row-parallel split)."""
    m = W.shape[0]
    assert m % N == 0
    w = m // N
    return np.ascontiguousarray(W[i * w:(i + 1) * w, :])


def mlp_inputs(M: int, h: int, f_full: int, N: int, dtype: str, seed: int,
               sigma_x: float = 1.0, sigma_w: float = 0.02, sigma_dz: float | None = 1.0,
               full: bool = True):
    """MLP workload.

    full=True draws the unsharded A [h, f_full] and B [f_full, h] and returns their
    N shards (so the sum over shards can be compared with the unsharded MLP).
    full=False draws only one rank's A_i [h, f_full] and B_i [f_full, h] (N=1 slice),
    used where the unsharded weights would not fit a test's time budget.
    Draw order: X, A, B, dZ. Returned arrays are float32 (dtype "f32") or
    bfloat16 bit patterns (uint16).
    """
    rng = np.random.default_rng(seed)
    X = _store(draw_normal_f32(rng, (M, h), sigma_x), dtype)
    A = _store(draw_normal_f32(rng, (h, f_full), sigma_w), dtype)
    B = _store(draw_normal_f32(rng, (f_full, h), sigma_w), dtype)
    dZ = None
    if sigma_dz is not None:
        dZ = _store(draw_normal_f32(rng, (M, h), sigma_dz), dtype)
    if full:
        shards = [(shard_cols(A, N, i), shard_rows(B, N, i)) for i in range(N)]
    else:
        shards = [(A, B)]
    return dict(X=X, A=A, B=B, dZ=dZ, shards=shards)


def attn_inputs(b: int, s: int, h: int, n_heads_local: int, d_head: int, seed: int,
                sigma_x: float = 1.0, sigma_w: float = 0.006):
    """Attention workload for one rank: X [b*s, h], Wqkv_i [h, 3*Hl*d], Wo_i [Hl*d, h].

    Wqkv_i columns are laid out [Q heads | K heads | V heads], local head j at
    columns j*d .. (j+1)*d of each block; Wo_i rows follow the same head order.
    Draw order: X, Wqkv_i, Wo_i. All bfloat16 bit patterns.
    """
    rng = np.random.default_rng(seed)
    X = bf16_bits(draw_normal_f32(rng, (b * s, h), sigma_x))
    Wqkv = bf16_bits(draw_normal_f32(rng, (h, 3 * n_heads_local * d_head), sigma_w))
    Wo = bf16_bits(draw_normal_f32(rng, (n_heads_local * d_head, h), sigma_w))
    return dict(X=X, Wqkv=Wqkv, Wo=Wo)


def embed_inputs(v: int, h: int, n_tokens: int, seed: int, sigma_w: float = 0.02,
                 chunk_rows: int = 4096):
    """Vocab-parallel embedding workload: full table E [v, h] (bf16 bits) drawn
    first, then token ids int32 uniform in [0, v). The table is drawn in row
    chunks to bound host memory; the stream of samples equals one big draw.
    Signed zeros are stored as +0.0."""
    rng = np.random.default_rng(seed)
    E = np.empty((v, h), np.uint16)
    for r0 in range(0, v, chunk_rows):
        r1 = min(v, r0 + chunk_rows)
        E[r0:r1] = bf16_bits(draw_normal_f32(rng, (r1 - r0, h), sigma_w))
    # numpy's float32 normal sampler returns exact zeros (with either sign) about
    # once per 2^23 draws; keep them as +0.0 so the sum of shards (which adds
    # +0.0 rows from the ranks that miss) reproduces the table bit for bit.
    E[E == 0x8000] = 0
    ids = rng.integers(0, v, size=n_tokens, dtype=np.int32)
    return dict(E=E, ids=ids)


def ce_inputs(M: int, h: int, v: int, seed: int, sigma_h: float = 1.0, sigma_w: float = 0.02,
              chunk_rows: int = 4096):
    """Output-layer + cross-entropy workload: final hidden rows H [M, h] (bf16
    bits), then the full word-embedding table E [v, h] (bf16 bits, drawn in row
    chunks like ``embed_inputs``), then target ids int32 uniform in [0, v)."""
    rng = np.random.default_rng(seed)
    H = bf16_bits(draw_normal_f32(rng, (M, h), sigma_h))
    E = np.empty((v, h), np.uint16)
    for r0 in range(0, v, chunk_rows):
        r1 = min(v, r0 + chunk_rows)
        E[r0:r1] = bf16_bits(draw_normal_f32(rng, (r1 - r0, h), sigma_w))
    targets = rng.integers(0, v, size=M, dtype=np.int32)
    return dict(H=H, E=E, targets=targets)


def sp_inputs(s: int, h: int, seed: int, sigma_r: float = 1.0, sigma_g: float = 0.1,
              sigma_b: float = 0.1, keep_prob: float = 0.9):
    """Sequence-parallel block inputs: residual rows R [s, h] float32 N(0, sigma_r),
    LayerNorm gamma = 1 + N(0, sigma_g) and beta = N(0, sigma_b) [h] float32, then a
    dropout keep mask [s, h] uint8 (1 where a uniform draw in [0, 1) is below keep_prob)."""
    rng = np.random.default_rng(seed)
    R = draw_normal_f32(rng, (s, h), sigma_r)
    gamma = (np.float32(1.0) + draw_normal_f32(rng, (h,), sigma_g)).astype(np.float32)
    beta = draw_normal_f32(rng, (h,), sigma_b)
    keep = (rng.random((s, h), dtype=np.float32) < np.float32(keep_prob)).astype(np.uint8)
    return dict(R=R, gamma=gamma, beta=beta, keep=keep)


def shard_sum_inputs(n_partials: int, numel: int, seed: int, sigma: float = 1.0,
                     dtype: str = "f32"):
    """N independent partials of numel elements, drawn in order 0..N-1."""
    rng = np.random.default_rng(seed)
    return [_store(draw_normal_f32(rng, (numel,), sigma), dtype) for _ in range(n_partials)]
