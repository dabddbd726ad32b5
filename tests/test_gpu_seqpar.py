"""GPU parity of the sequence-parallel kernels (LayerNorm on a rank's rows, the
all-gather and reduce-scatter stand-ins, dropout + residual) and of the whole
sequence-parallel MLP block against the float64 oracle, through the C ABI.

Tolerances: LayerNorm runs in float32 and rounds once to bf16, so each output is
within one bf16 spacing of the float64 value (plus 4e-6 for the float32
arithmetic near zero, whose terms are O(1)); the all-gather is a copy
(bit-exact); the reduce-scatter adds N float32 values in rank order, so it is
within 1e-5 absolute + 1e-6 relative of the float64 sum, and dropped entries
equal the residual exactly. The block's MLP uses the bf16 GEMM tolerance.
"""
import numpy as np
import pytest
import torch

import oracle
from oracle import seqpar
from tests.gpu_util import DEV, assert_bf16_close, bits_host, f32_dev, f64_host, note
from workloads import CONFIGS, mlp_inputs, shard_sum_inputs, sp_inputs

pytestmark = pytest.mark.gpu

tp = pytest.importorskip("attention_shard_math_amd")


def _bf16_spacing(r):
    a = np.maximum(np.abs(r), np.finfo(np.float32).tiny)
    return np.exp2(np.floor(np.log2(a)) - 7)


def assert_ln_close(g, r, what):
    d = np.abs(g - r)
    bad = d > _bf16_spacing(r) + 4e-6
    assert not bad.any(), f"{what}: {bad.sum()} outputs beyond one bf16 spacing (max diff {d.max():.3e})"
    same = np.mean(g == oracle.round_to_bf16(r))
    assert same >= 0.99, f"{what}: only {same:.4f} equal the rounded float64 value"


def _ln_gpu(R, gamma, beta):
    rows, h = R.shape
    Y = torch.empty(rows, h, dtype=torch.bfloat16, device=DEV)
    tp.layernorm(f32_dev(R), f32_dev(gamma), f32_dev(beta), Y)
    return Y


@pytest.mark.parametrize("rows,h", [(37, 8), (5, 328), (64, 1032), (3, 12288), (2, 18432), (1, 32768)])
def test_layernorm(rows, h):
    inp = sp_inputs(rows, h, seed=500 + h, sigma_r=2.0)
    R = inp["R"] + np.float32(0.75)  # a row mean away from zero
    note(f"layernorm rows={rows} h={h}")
    Y = _ln_gpu(R, inp["gamma"], inp["beta"])
    torch.cuda.synchronize()
    r = seqpar.layernorm(R.astype(np.float64), inp["gamma"], inp["beta"])
    assert_ln_close(f64_host(Y), r, f"LN rows={rows} h={h}")


def test_layernorm_constant_row_gives_beta():
    h = 256
    R = np.full((3, h), 2.5, np.float32)
    gamma = np.linspace(0.5, 1.5, h, dtype=np.float32)
    beta = np.linspace(-1, 1, h, dtype=np.float32)
    note("layernorm constant rows")
    Y = _ln_gpu(R, gamma, beta)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(f64_host(Y), np.broadcast_to(oracle.round_to_bf16(beta.astype(np.float64)), (3, h)))


def test_all_gather_bit_exact():
    for n, rows, h in [(1, 3, 8), (4, 17, 64), (16, 2, 1024)]:
        note(f"sp_all_gather n={n} rows={rows} h={h}")
        sl = [torch.randn(rows, h, device=DEV).to(torch.bfloat16) for _ in range(n)]
        out = torch.empty(n * rows, h, dtype=torch.bfloat16, device=DEV)
        tp.sp_all_gather(sl, out)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(bits_host(out), np.concatenate([bits_host(x) for x in sl]))


@pytest.mark.parametrize("n,s,h,drop", [(1, 4, 8, False), (3, 30, 72, True), (8, 64, 520, True), (16, 32, 64, False)])
def test_reduce_scatter(n, s, h, drop):
    parts = [p.reshape(s, h) for p in shard_sum_inputs(n, s * h, seed=600 + n)]
    inp = sp_inputs(s, h, seed=700 + n, keep_prob=0.8)
    rows = s // n
    pd = [f32_dev(p) for p in parts]
    for rank in sorted({0, n // 2, n - 1}):
        rs = slice(rank * rows, (rank + 1) * rows)
        keep = inp["keep"][rs] if drop else None
        note(f"sp_reduce_scatter n={n} s={s} h={h} rank={rank} dropout={drop}")
        out = torch.full((rows, h), float("nan"), dtype=torch.float32, device=DEV)
        tp.sp_reduce_scatter(pd, rank, f32_dev(inp["R"][rs]), out,
                             keep=None if keep is None else torch.from_numpy(keep).to(DEV), keep_prob=0.8)
        torch.cuda.synchronize()
        O = seqpar.reduce_scatter(parts, n, rank)
        want = seqpar.dropout_residual(inp["R"][rs], O, keep, 0.8)
        g = f64_host(out)
        np.testing.assert_allclose(g, want, rtol=1e-6, atol=1e-5)
        if drop:
            np.testing.assert_array_equal(g[keep == 0], inp["R"][rs][keep == 0])


def test_reduce_scatter_in_place():
    n, s, h = 4, 16, 64
    parts = [p.reshape(s, h) for p in shard_sum_inputs(n, s * h, seed=611)]
    R = sp_inputs(s, h, seed=612)["R"]
    note("sp_reduce_scatter in place")
    res = f32_dev(R[4:8])
    tp.sp_reduce_scatter([f32_dev(p) for p in parts], 1, res, res)
    torch.cuda.synchronize()
    np.testing.assert_allclose(f64_host(res), R[4:8] + seqpar.reduce_scatter(parts, n, 1), rtol=1e-6, atol=1e-5)


def _sp_block_gpu(R, gamma, beta, shards_dev, keep, p, N):
    s, h = R.shape
    rows = s // N
    Rd, g, b = f32_dev(R), f32_dev(gamma), f32_dev(beta)
    L = [torch.empty(rows, h, dtype=torch.bfloat16, device=DEV) for _ in range(N)]
    for i in range(N):
        tp.layernorm(Rd[i * rows:(i + 1) * rows], g, b, L[i])
    X = torch.empty(s, h, dtype=torch.bfloat16, device=DEV)
    tp.sp_all_gather(L, X)
    Z = []
    for A, B in shards_dev:
        f = A.shape[1]
        Y = torch.empty(s, f, dtype=torch.bfloat16, device=DEV)
        z = torch.empty(s, h, dtype=torch.float32, device=DEV)
        tp.mlp_fwd(X, A, B, Y, z)
        Z.append(z)
    out = torch.empty(s, h, dtype=torch.float32, device=DEV)
    kd = torch.from_numpy(keep).to(DEV)
    for i in range(N):
        rs = slice(i * rows, (i + 1) * rows)
        tp.sp_reduce_scatter(Z, i, Rd[rs], out[rs], keep=kd[rs], keep_prob=p)
    return X, out


@pytest.mark.parametrize("N", [2, 4])
def test_sp_mlp_block(N):
    s, h, f_full = 256, 1024, 4096
    sp = sp_inputs(s, h, seed=800 + N, keep_prob=0.9)
    mi = mlp_inputs(s, h, f_full, N, "bf16", 810 + N, 1.0, 0.02, None)
    from tests.gpu_util import bf16_dev
    from oracle.bf16 import bf16_bits_to_f64
    shards_dev = [(bf16_dev(A), bf16_dev(B)) for A, B in mi["shards"]]
    note(f"sequence-parallel MLP block s={s} h={h} N={N}")
    X, out = _sp_block_gpu(sp["R"], sp["gamma"], sp["beta"], shards_dev, sp["keep"], 0.9, N)
    torch.cuda.synchronize()
    shards = [(bf16_bits_to_f64(A), bf16_bits_to_f64(B)) for A, B in mi["shards"]]
    R64 = sp["R"].astype(np.float64)
    want = seqpar.sp_mlp_block(R64, sp["gamma"], sp["beta"], shards, sp["keep"], 0.9, matched=True)
    assert_ln_close(f64_host(X), seqpar.layernorm(R64, sp["gamma"], sp["beta"]), "gathered LN")
    assert_bf16_close(f64_host(out) - R64, want["R_out"] - R64, "dropout(reduce-scatter)")


def test_full_size_layernorm_gather_reduce_scatter():
    """GPT-3 shard: 8 ranks of 256 rows x 12288; the reduce-scatter of 8 fp32
    partials [2048, 12288] with dropout 0.9 and the residual, for every rank."""
    c = CONFIGS["gpt3_sp_mlp_block"]
    s, h, N = c["s"], c["h"], c["N"]
    rows = s // N
    sp = sp_inputs(s, h, c["seed"], c["sigma_r"], c["sigma_g"], c["sigma_b"], c["keep_prob"])
    parts = [p.reshape(s, h) for p in shard_sum_inputs(N, s * h, c["seed"] + 1, c["sigma_p"])]
    Rd, g, b = f32_dev(sp["R"]), f32_dev(sp["gamma"]), f32_dev(sp["beta"])
    L = [torch.empty(rows, h, dtype=torch.bfloat16, device=DEV) for _ in range(N)]
    note("full-size layernorm x8 + all-gather")
    for i in range(N):
        tp.layernorm(Rd[i * rows:(i + 1) * rows], g, b, L[i])
    X = torch.empty(s, h, dtype=torch.bfloat16, device=DEV)
    tp.sp_all_gather(L, X)
    torch.cuda.synchronize()
    assert_ln_close(f64_host(X), seqpar.layernorm(sp["R"].astype(np.float64), sp["gamma"], sp["beta"]), "LN 2048x12288")
    pd = [f32_dev(p) for p in parts]
    kd = torch.from_numpy(sp["keep"]).to(DEV)
    out = torch.empty(s, h, dtype=torch.float32, device=DEV)
    note("full-size reduce-scatter x8")
    for i in range(N):
        rs = slice(i * rows, (i + 1) * rows)
        tp.sp_reduce_scatter(pd, i, Rd[rs], out[rs], keep=kd[rs], keep_prob=c["keep_prob"])
    torch.cuda.synchronize()
    g_out = f64_host(out)
    for i in range(N):
        rs = slice(i * rows, (i + 1) * rows)
        want = seqpar.dropout_residual(sp["R"][rs], seqpar.reduce_scatter(parts, N, i), sp["keep"][rs], c["keep_prob"])
        np.testing.assert_allclose(g_out[rs], want, rtol=1e-6, atol=1e-5)


# ---------------------------------------------------------------- backward
# LayerNorm's backward is float32 throughout: dX within 2e-5 of max|dX| plus 1e-4
# relative per element, dgamma/dbeta (sums over the rows) within 1e-4 relative
# plus 1e-5 of their maximum. Dropout's backward rounds once to bf16: within one
# bf16 spacing of the float64 value.


def _close_f32(g, r, what, rel=1e-4, nw=2e-5):
    g, r = np.asarray(g, np.float64), np.asarray(r, np.float64)
    assert np.all(np.isfinite(g)), f"{what}: non-finite"
    tol = rel * np.abs(r) + nw * max(np.abs(r).max(), 1e-30)
    bad = np.abs(g - r) > tol
    assert not bad.any(), f"{what}: {bad.sum()} beyond tolerance, max diff {np.abs(g - r).max():.3e}"


def _close_rel(g, r, what):
    """The bf16-GEMM bar of every product: max|g - r| <= 2e-2 max|r| and
    mean|g - r| <= 1e-3, against the matched oracle."""
    assert_bf16_close(g, r, what)


def _ln_bwd_gpu(R, gamma, dY, dRes=None):
    rows, h = R.shape
    dX = torch.full((rows, h), float("nan"), dtype=torch.float32, device=DEV)
    dg = torch.full((h,), float("nan"), dtype=torch.float32, device=DEV)
    db = torch.full((h,), float("nan"), dtype=torch.float32, device=DEV)
    ws = torch.empty(tp.layernorm_bwd_workspace(rows, h), dtype=torch.uint8, device=DEV)
    tp.layernorm_bwd(f32_dev(R), f32_dev(gamma), f32_dev(dY), dX, dg, db, ws,
                     dRes=None if dRes is None else f32_dev(dRes))
    return dX, dg, db


@pytest.mark.parametrize("rows,h,res", [(37, 8, False), (5, 328, True), (64, 1032, False), (3, 12288, True),
                                        (2, 18432, False), (100, 24576, False), (256, 12288, True)])
def test_layernorm_bwd(rows, h, res):
    inp = sp_inputs(rows, h, seed=900 + h + rows, sigma_r=2.0)
    rng = np.random.default_rng(901 + h)
    dY = rng.standard_normal((rows, h)).astype(np.float32)
    dRes = rng.standard_normal((rows, h)).astype(np.float32) if res else None
    R = inp["R"] + np.float32(0.5)
    note(f"layernorm_bwd rows={rows} h={h} dRes={res}")
    dX, dg, db = _ln_bwd_gpu(R, inp["gamma"], dY, dRes)
    torch.cuda.synchronize()
    r = seqpar.layernorm_bwd(R.astype(np.float64), inp["gamma"], dY)
    want = r["dX"] + (dRes if res else 0.0)
    _close_f32(f64_host(dX), want, "dX")
    _close_f32(f64_host(dg), r["dgamma"], "dgamma")
    _close_f32(f64_host(db), r["dbeta"], "dbeta")


@pytest.mark.parametrize("rows,h", [(256, 12288), (100, 1032), (5, 8)])
def test_layernorm_bwd_is_deterministic(rows, h):
    """dgamma and dbeta are sums over the rows in a fixed order: two calls give the
    same bits, whatever the workspace held before."""
    note(f"layernorm_bwd determinism rows={rows} h={h}")
    inp = sp_inputs(rows, h, seed=950 + rows, sigma_r=2.0)
    rng = np.random.default_rng(951 + h)
    dY = f32_dev(rng.standard_normal((rows, h)).astype(np.float32))
    R, g = f32_dev(inp["R"]), f32_dev(inp["gamma"])
    ws = torch.empty(tp.layernorm_bwd_workspace(rows, h), dtype=torch.uint8, device=DEV)
    outs = []
    for fill in (0x00, 0x7F):
        ws.fill_(fill)
        dX = torch.empty(rows, h, dtype=torch.float32, device=DEV)
        dg = torch.empty(h, dtype=torch.float32, device=DEV)
        db = torch.empty(h, dtype=torch.float32, device=DEV)
        tp.layernorm_bwd(R, g, dY, dX, dg, db, ws)
        torch.cuda.synchronize()
        outs.append((dX, dg, db))
    for a, b_ in zip(*outs):
        assert torch.equal(a.view(torch.int32), b_.view(torch.int32))


def test_dropout_bwd():
    for rows, h, drop in [(3, 8, False), (17, 72, True), (256, 12288, True)]:
        note(f"sp_dropout_bwd rows={rows} h={h} dropout={drop}")
        rng = np.random.default_rng(950 + h)
        dY = rng.standard_normal((rows, h)).astype(np.float32)
        keep = (rng.random((rows, h)) < 0.9).astype(np.uint8) if drop else None
        out = torch.empty(rows, h, dtype=torch.bfloat16, device=DEV)
        tp.sp_dropout_bwd(f32_dev(dY), out, keep=None if keep is None else torch.from_numpy(keep).to(DEV),
                          keep_prob=0.9)
        torch.cuda.synchronize()
        r = seqpar.dropout_bwd(dY, keep, 0.9)
        g = f64_host(out)
        assert np.all(np.abs(g - r) <= _bf16_spacing(r)), "dropout_bwd beyond one bf16 spacing"
        if drop:
            assert np.all(g[keep == 0] == 0.0)


@pytest.mark.parametrize("N", [2, 4])
def test_sp_mlp_block_backward(N):
    """The whole sequence-parallel block backward composed from the C ABI:
    dropout backward -> all-gather -> MLP backward per rank -> reduce-scatter ->
    LayerNorm backward with the residual path, against the float64 oracle."""
    s, h, f_full, p = 256, 1024, 4096, 0.9
    sp = sp_inputs(s, h, seed=960 + N, keep_prob=p)
    mi = mlp_inputs(s, h, f_full, N, "bf16", 970 + N, 1.0, 0.02, None)
    dRo = np.random.default_rng(980 + N).standard_normal((s, h)).astype(np.float32)
    from tests.gpu_util import bf16_dev
    from oracle.bf16 import bf16_bits_to_f64
    rows = s // N
    note(f"sequence-parallel block backward s={s} h={h} N={N}")
    shards_dev = [(bf16_dev(A), bf16_dev(B)) for A, B in mi["shards"]]
    X, _ = _sp_block_gpu(sp["R"], sp["gamma"], sp["beta"], shards_dev, sp["keep"], p, N)
    kd = torch.from_numpy(sp["keep"]).to(DEV)
    dRd = f32_dev(dRo)
    sl = [torch.empty(rows, h, dtype=torch.bfloat16, device=DEV) for _ in range(N)]
    for i in range(N):
        rs = slice(i * rows, (i + 1) * rows)
        tp.sp_dropout_bwd(dRd[rs], sl[i], keep=kd[rs], keep_prob=p)
    dZ = torch.empty(s, h, dtype=torch.bfloat16, device=DEV)
    tp.sp_all_gather(sl, dZ)
    dXp, dAs, dBs = [], [], []
    for A, B in shards_dev:
        f = A.shape[1]
        U = torch.empty(s, f, dtype=torch.bfloat16, device=DEV)
        Y = torch.empty(s, f, dtype=torch.bfloat16, device=DEV)
        Z = torch.empty(s, h, dtype=torch.float32, device=DEV)
        tp.mlp_fwd(X, A, B, Y, Z, U_i=U)
        dX = torch.empty(s, h, dtype=torch.float32, device=DEV)
        dA = torch.empty(h, f, dtype=torch.float32, device=DEV)
        dB = torch.empty(f, h, dtype=torch.float32, device=DEV)
        ws = torch.empty(tp.mlp_bwd_workspace(s, h, f), dtype=torch.uint8, device=DEV)
        tp.mlp_bwd(X, A, B, U, Y, dZ, dX, dA, dB, ws)
        dXp.append(dX)
        dAs.append(dA)
        dBs.append(dB)
    Rd, gd = f32_dev(sp["R"]), f32_dev(sp["gamma"])
    dR = torch.empty(s, h, dtype=torch.float32, device=DEV)
    dgs, dbs = [], []
    lws = torch.empty(tp.layernorm_bwd_workspace(rows, h), dtype=torch.uint8, device=DEV)
    for i in range(N):
        rs = slice(i * rows, (i + 1) * rows)
        dL = torch.empty(rows, h, dtype=torch.float32, device=DEV)
        tp.sp_reduce_scatter(dXp, i, None, dL)
        dg = torch.empty(h, dtype=torch.float32, device=DEV)
        db = torch.empty(h, dtype=torch.float32, device=DEV)
        tp.layernorm_bwd(Rd[rs], gd, dL, dR[rs], dg, db, lws, dRes=dRd[rs])
        dgs.append(dg)
        dbs.append(db)
    dgam = torch.empty(h, dtype=torch.float32, device=DEV)
    dbet = torch.empty(h, dtype=torch.float32, device=DEV)
    tp.shard_sum(dgs, dgam)
    tp.shard_sum(dbs, dbet)
    torch.cuda.synchronize()
    shards = [(bf16_bits_to_f64(A), bf16_bits_to_f64(B)) for A, B in mi["shards"]]
    want = seqpar.sp_mlp_block_bwd(sp["R"].astype(np.float64), sp["gamma"], sp["beta"], shards, dRo, sp["keep"], p,
                                   matched=True)
    _close_rel(f64_host(dZ), want["dZ"], "gathered dZ")
    _close_rel(f64_host(dR) - dRo, want["dR"] - dRo, "dR (through LayerNorm)")
    _close_rel(f64_host(dgam), want["dgamma"], "dgamma")
    _close_rel(f64_host(dbet), want["dbeta"], "dbeta")
    for j in range(N):
        _close_rel(f64_host(dAs[j]), want["dA"][j], f"dA_{j}")
        _close_rel(f64_host(dBs[j]), want["dB"][j], f"dB_{j}")
