"""The allocation-free MLP backward (tp_mlp_bwd_noalloc), for callers that cannot
allocate: through the C ABI, two calls in a row on one device (the second with a
smaller problem, so the shared scratch still holds the first call's dU), each
against tp_mlp_bwd with a caller workspace on the same inputs, at the bf16 bar
(normwise 2e-2, mean abs 1e-3). Both run the same four products, but tp_mlp_bwd
may split a product's k-range over the workgroups (stream-K) where the no-alloc
variant runs one tile per workgroup: the bf16 dU then rounds differently in a few
entries, and dX, dA that are formed from it differ by more than float32 rounding."""
import numpy as np
import pytest
import torch

from tests.gpu_util import DEV, assert_bf16_close, bf16_dev, note
from workloads import mlp_inputs

pytestmark = pytest.mark.gpu

tp = pytest.importorskip("attention_shard_math_amd")


def _run(M, h, f, seed, noalloc):
    inp = mlp_inputs(M, h, f, 1, "bf16", seed, 1.0, 0.02, 1.0, full=False)
    X, A, B, dZ = (bf16_dev(inp[k]) for k in ("X", "A", "B", "dZ"))
    U = torch.empty(M, f, dtype=torch.bfloat16, device=DEV)
    Y = torch.empty(M, f, dtype=torch.bfloat16, device=DEV)
    Z = torch.empty(M, h, dtype=torch.float32, device=DEV)
    tp.mlp_fwd(X, A, B, Y, Z, U_i=U)
    outs = [torch.full(shape, float("nan"), dtype=torch.float32, device=DEV) for shape in ((M, h), (h, f), (f, h))]
    if noalloc:
        tp.mlp_bwd_noalloc(X, A, B, U, Y, dZ, *outs)
    else:
        ws = torch.empty(tp.mlp_bwd_workspace(M, h, f), dtype=torch.uint8, device=DEV)
        tp.mlp_bwd(X, A, B, U, Y, dZ, *outs, ws)
    torch.cuda.synchronize()
    return [o.double().cpu().numpy() for o in outs]


def test_noalloc_matches_workspace_call_twice():
    for (M, h, f, seed) in [(1000, 1024, 2048, 31), (200, 512, 768, 32)]:
        note(f"mlp_bwd_noalloc M={M} h={h} f={f}")
        got = _run(M, h, f, seed, True)
        note(f"mlp_bwd (workspace) M={M} h={h} f={f}")
        want = _run(M, h, f, seed, False)
        for g, r, name in zip(got, want, ("dX_i", "dA_i", "dB_i")):
            assert np.all(np.isfinite(g)), name
            assert_bf16_close(g, r, f"{name} M={M}")
