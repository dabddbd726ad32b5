"""CPU oracle for the rank-shard tensor-parallel path — TEST INFRASTRUCTURE ONLY.

A plain, slow, float64 reference of what one tensor-parallel rank computes in a
Megatron-style Transformer layer. It exists to check the HIP path and nothing
else: only the test suite, the smoke check and the benchmark's CPU-baseline leg
may import it. The product path never calls it and has no CPU fallback.

It shares no code with the HIP library: numpy (float64 BLAS), scipy's erf and
Python loops only. Every function cites the passage of the pages it follows.

Pages cited (by title and section as printed):
  * "Megatron-LM：张量并行与大规模训练" (astro-blog-cod.pages.dev) — §2.1 MLP 层的
    张量并行 (column split of A, row split of B, the partial sums Z_i and their
    all-reduce), §2.2 Self-Attention 的张量并行 (heads split across ranks,
    row-parallel output projection), §5.5 BF16 vs FP16 (the bf16 format),
    §5.6 GPT-3 (175B) 的训练配置 (the shapes).
  * m.youleyou.com/wenzhang/3143730 (untitled in the extract) — 一、切分权重 §1.1/§1.2
    (row and column splits with the conjugate f/g operators, forward and
    backward), 二、MLP层 §2.1, 三、Self-Attention层 §3.1, 四、Embedding层 §4.1
    (vocabulary-parallel input embedding with zeroed misses), §4.2 and
    五、Cross-Entropy层 (vocabulary-parallel output layer and loss), 二、§2.2
    (an all-reduce is a reduce-scatter plus an all-gather).
  * www.discosf.com/news/5875844 — 2.3 序列并行与激活重计算 (sequence-parallel
    LayerNorm and Dropout; activation recompute).
  * "Megatron-LM 介绍" (apxml.com) — 核心贡献 item 1 (ColumnParallelLinear).

Parity status per function (what pins it, see tests/test_oracle_pins.py):
  bf16 rounding, GeLU/GeLU', MLP forward/backward, shard-sum, attention, the
  embedding gather, the vocabulary-parallel cross-entropy and the
  sequence-parallel LayerNorm / reduce-scatter / all-gather / dropout are each
  pinned by closed forms, brute force on tiny inputs,
  finite differences, sharding invariants or the pages' worked example. No
  function is "parity unpinned".
"""
from .bf16 import round_to_bf16, bf16_bits_to_f64, f64_to_bf16_bits  # noqa: F401
from .mlp import (  # noqa: F401
    gelu, gelu_prime, mlp_fwd_shard, mlp_bwd_shard, mlp_fwd_full, mlp_bwd_full,
    mlp_fwd_rows, mlp_bwd_cols,
)
from .shard_sum import shard_sum_f64, shard_sum_f32_ordered, shard_sum_bf16_ordered  # noqa: F401
from .attention import (  # noqa: F401
    attn_shard, attn_core, mha_full, attn_shard_rows, attn_core_bwd, attn_lse, attn_shard_bwd,
)
from .embedding import vocab_embed_shard  # noqa: F401
from .vocab_ce import vocab_ce_partials, vocab_ce_combine, vocab_ce_sharded  # noqa: F401
from .seqpar import (  # noqa: F401
    layernorm, all_gather, reduce_scatter, dropout_residual, sp_mlp_block, tp_mlp_block, layernorm_bwd,
    dropout_bwd, sp_mlp_block_bwd,
)
