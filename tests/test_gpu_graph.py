"""The C ABI is capture-safe: no allocation, no synchronisation and no memset
inside any call, so a whole training step of the rank shard (MLP, attention,
shard-sum and the sequence-parallel kernels) can be recorded in a HIP graph
(through torch.cuda.graph) and replayed. Every replay, with eager
work and synchronisations in between, must reproduce the eager results bit for
bit (the kernels are deterministic)."""
import numpy as np
import pytest
import torch

from tests.gpu_util import DEV, bf16_dev, note
from workloads import attn_inputs, bf16_bits, draw_normal_f32, mlp_inputs

pytestmark = pytest.mark.gpu

tp = pytest.importorskip("attention_shard_math_amd")


def test_step_in_a_graph_replays_bit_exactly():
    M, h, f = 256, 512, 768
    inp = mlp_inputs(M, h, f, 1, "bf16", 31, 1.0, 0.05, 1.0, full=False)
    A_i, B_i = inp["shards"][0]
    X, A, B, dZ = bf16_dev(inp["X"]), bf16_dev(A_i), bf16_dev(B_i), bf16_dev(inp["dZ"])
    b, s, Hl, d = 1, 256, 2, 128
    ai = attn_inputs(b, s, h, Hl, d, 32, 1.0, 0.05)
    Xa, Wqkv, Wo = (bf16_dev(ai[k]) for k in ("X", "Wqkv", "Wo"))
    dOut = bf16_dev(bf16_bits(draw_normal_f32(np.random.default_rng(33), (b * s, h), 1.0)))
    w = Hl * d

    U = torch.empty(M, f, dtype=torch.bfloat16, device=DEV)
    Y = torch.empty_like(U)
    Z = torch.empty(M, h, dtype=torch.float32, device=DEV)
    dX = torch.empty(M, h, dtype=torch.float32, device=DEV)
    dA = torch.empty(h, f, dtype=torch.float32, device=DEV)
    dB = torch.empty(f, h, dtype=torch.float32, device=DEV)
    ws = torch.empty(tp.mlp_bwd_workspace(M, h, f), dtype=torch.uint8, device=DEV)
    out = torch.empty(b * s, h, dtype=torch.float32, device=DEV)
    QKV = torch.empty(b * s, 3 * w, dtype=torch.bfloat16, device=DEV)
    O = torch.empty(b * s, w, dtype=torch.bfloat16, device=DEV)
    lse = torch.empty(b, Hl, s, dtype=torch.float32, device=DEV)
    dXa = torch.empty(b * s, h, dtype=torch.float32, device=DEV)
    dWqkv = torch.empty(h, 3 * w, dtype=torch.float32, device=DEV)
    dWo = torch.empty(w, h, dtype=torch.float32, device=DEV)
    wsb = torch.empty(tp.attn_bwd_workspace(b, s, h, Hl, d), dtype=torch.uint8, device=DEV)
    tot = torch.empty(M, h, dtype=torch.float32, device=DEV)
    # sequence-parallel kernels: 2 ranks of 128 rows over the same h
    rng = np.random.default_rng(34)
    Rs = torch.from_numpy(draw_normal_f32(rng, (128, h), 1.0)).to(DEV)
    gam = torch.from_numpy(draw_normal_f32(rng, (h,), 0.1)).to(DEV) + 1.0
    bet = torch.from_numpy(draw_normal_f32(rng, (h,), 0.1)).to(DEV)
    dYs = torch.from_numpy(draw_normal_f32(rng, (128, h), 1.0)).to(DEV)
    keep = torch.from_numpy((rng.random((128, h)) < 0.9).astype(np.uint8)).to(DEV)
    Ln = torch.empty(128, h, dtype=torch.bfloat16, device=DEV)
    Lg = torch.empty(256, h, dtype=torch.bfloat16, device=DEV)
    Ro = torch.empty(128, h, dtype=torch.float32, device=DEV)
    dXs = torch.empty(128, h, dtype=torch.float32, device=DEV)
    dgs = torch.empty(h, dtype=torch.float32, device=DEV)
    dbs = torch.empty(h, dtype=torch.float32, device=DEV)
    dZs = torch.empty(128, h, dtype=torch.bfloat16, device=DEV)
    lws = torch.empty(tp.layernorm_bwd_workspace(128, h), dtype=torch.uint8, device=DEV)
    outs = (U, Y, Z, dX, dA, dB, out, QKV, O, lse, dXa, dWqkv, dWo, tot, Ln, Lg, Ro, dXs, dgs, dbs, dZs)

    def step():
        tp.mlp_fwd(X, A, B, Y, Z, U_i=U)
        tp.mlp_bwd(X, A, B, U, Y, dZ, dX, dA, dB, ws)
        tp.attn_fwd_train(Xa, Wqkv, Wo, out, QKV, O, lse, b, s, Hl, d, True)
        tp.attn_bwd(Xa, Wqkv, Wo, QKV, O, lse, dOut, dXa, dWqkv, dWo, wsb, b, s, Hl, d, True)
        tp.shard_sum([Z, dX], tot)
        tp.layernorm(Rs, gam, bet, Ln)
        tp.sp_all_gather([Ln, Ln], Lg)
        tp.sp_reduce_scatter([Z[:256], dX[:256]], 1, Rs, Ro, keep=keep, keep_prob=0.9)
        tp.layernorm_bwd(Rs, gam, dYs, dXs, dgs, dbs, lws, dRes=Ro)
        tp.sp_dropout_bwd(dYs, dZs, keep=keep, keep_prob=0.9)

    note("graph: eager step")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    want = [t.clone() for t in outs]

    note("graph: capture")
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for r in range(3):
        for t in outs:
            t.fill_(float("nan")) if t.dtype.is_floating_point else t.zero_()
        torch.cuda.synchronize()
        note(f"graph: replay {r}")
        graph.replay()
        torch.cuda.synchronize()
        for name, g, e in zip(("U", "Y", "Z", "dX", "dA", "dB", "out", "QKV", "O", "lse", "dXa", "dWqkv", "dWo",
                               "sum", "ln", "gather", "rs", "ln dX", "dgamma", "dbeta", "dropout dY"), outs, want):
            assert torch.equal(g.view(torch.uint8), e.view(torch.uint8)), f"replay {r}: {name} differs"
