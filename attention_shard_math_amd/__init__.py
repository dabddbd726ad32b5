"""attention_shard_math_amd — Python binding of libtpshard, one tensor-parallel
rank's shard of a Megatron-style Transformer layer on MI355X.

Argument marshalling only: every step runs in the HIP kernels of libtpshard.so
(built in-tree by ``attention_shard_math_amd.build``). Torch tensors supply
device memory and the current stream. There is no CPU fallback: importing the
package without the built library raises.
"""
from ._lib import (  # noqa: F401
    LIB_PATH,
    TpError,
    lib,
    column_linear,
    row_linear,
    linear_workspace,
    mlp_fwd,
    mlp_fwd_workspace,
    mlp_bwd,
    mlp_bwd_workspace,
    mlp_bwd_recompute_workspace,
    mlp_bwd_noalloc,
    mlp_bwd_noalloc_max_bytes,
    attn_core,
    attn_fwd,
    attn_fwd_workspace,
    attn_fwd_train,
    attn_core_train,
    attn_core_bwd,
    attn_core_bwd_workspace,
    attn_bwd,
    attn_bwd_workspace,
    vocab_embed,
    vocab_ce_workspace,
    vocab_ce_partials,
    vocab_ce_loss,
    shard_sum,
    layernorm,
    layernorm_bwd,
    layernorm_bwd_workspace,
    sp_dropout_bwd,
    sp_all_gather,
    sp_reduce_scatter,
)
