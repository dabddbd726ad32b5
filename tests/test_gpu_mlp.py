"""GPU parity of the MLP shard (column GEMM + GeLU, row GEMM, backward) against
the float64 oracle, through the C ABI."""
import numpy as np
import pytest
import torch

import oracle
from oracle.bf16 import bf16_bits_to_f64
from tests.gpu_util import (DEV, assert_bf16_close, assert_f32_close, bf16_dev, f32_dev, f64_host, note)
from workloads import CONFIGS, bf16_bits, mlp_inputs, shard_sum_inputs

pytestmark = pytest.mark.gpu

tp = pytest.importorskip("attention_shard_math_amd")


def _alloc(M, h, f, dt):
    U = torch.empty(M, f, dtype=dt, device=DEV)
    Y = torch.empty(M, f, dtype=dt, device=DEV)
    Z = torch.empty(M, h, dtype=torch.float32, device=DEV)
    return U, Y, Z


def _run_bwd(X, A, B, U, Y, dZ, M, h, f):
    ws = torch.empty(max(tp.mlp_bwd_workspace(M, h, f), 1), dtype=torch.uint8, device=DEV)
    dX = torch.full((M, h), float("nan"), dtype=torch.float32, device=DEV)
    dA = torch.full((h, f), float("nan"), dtype=torch.float32, device=DEV)
    dB = torch.full((f, h), float("nan"), dtype=torch.float32, device=DEV)
    tp.mlp_bwd(X, A, B, U, Y, dZ, dX, dA, dB, ws)
    return dX, dA, dB, ws


def test_tiny_mlp_fp32_two_shards():
    c = CONFIGS["tiny_mlp_fp32"]
    M = c["b"] * c["s"]
    inp = mlp_inputs(M, c["h"], c["f_full"], c["N"], "f32", c["seed"], c["sigma_x"], c["sigma_w"], None)
    note("tiny fp32 mlp_fwd, 2 shards")
    X = f32_dev(inp["X"])
    Zs = []
    for i, (A_i, B_i) in enumerate(inp["shards"]):
        f = A_i.shape[1]
        U, Y, Z = _alloc(M, c["h"], f, torch.float32)
        tp.mlp_fwd(X, f32_dev(A_i), f32_dev(B_i), Y, Z, U_i=U)
        torch.cuda.synchronize()
        r = oracle.mlp_fwd_shard(inp["X"].astype(np.float64), A_i.astype(np.float64), B_i.astype(np.float64),
                                 matched=False)
        assert_f32_close(f64_host(U), r["U"], f"U_{i}")
        assert_f32_close(f64_host(Y), r["Y"], f"Y_{i}")
        assert_f32_close(f64_host(Z), r["Z"], f"Z_{i}")
        Zs.append(Z)
    tot = torch.empty_like(Zs[0])
    tp.shard_sum(Zs, tot)
    torch.cuda.synchronize()
    full = oracle.mlp_fwd_full(*(inp[k].astype(np.float64) for k in "XAB"))
    assert_f32_close(f64_host(tot), full, "Z_1 + Z_2")


def _bf16_mlp_case(M, h, f_full, N, seed, sigma_w, check_unsharded=True):
    inp = mlp_inputs(M, h, f_full, N, "bf16", seed, 1.0, sigma_w, 1.0)
    X, dZ = bf16_dev(inp["X"]), bf16_dev(inp["dZ"])
    Xo, dZo = bf16_bits_to_f64(inp["X"]), bf16_bits_to_f64(inp["dZ"])
    Zs, dXs = [], []
    for i, (A_i, B_i) in enumerate(inp["shards"]):
        f = A_i.shape[1]
        note(f"bf16 mlp M={M} h={h} f={f} shard {i}/{N}")
        A, B = bf16_dev(A_i), bf16_dev(B_i)
        U, Y, Z = _alloc(M, h, f, torch.bfloat16)
        tp.mlp_fwd(X, A, B, Y, Z, U_i=U)
        dX, dA, dB, _ = _run_bwd(X, A, B, U, Y, dZ, M, h, f)
        torch.cuda.synchronize()
        Ao, Bo = bf16_bits_to_f64(A_i), bf16_bits_to_f64(B_i)
        r = oracle.mlp_fwd_shard(Xo, Ao, Bo)
        g = oracle.mlp_bwd_shard(Xo, Ao, Bo, r["U"], r["Y"], dZo)
        assert_bf16_close(f64_host(U), r["U"], f"U_{i}")
        assert_bf16_close(f64_host(Y), r["Y"], f"Y_{i}")
        assert_bf16_close(f64_host(Z), r["Z"], f"Z_{i}")
        assert_bf16_close(f64_host(dA), g["dA"], f"dA_{i}")
        assert_bf16_close(f64_host(dB), g["dB"], f"dB_{i}")
        assert_bf16_close(f64_host(dX), g["dX"], f"dX_{i}")
        Zs.append((Z, r["Z"]))
        dXs.append((dX, g["dX"]))
    for name, parts in (("Z", Zs), ("dX", dXs)):
        out = torch.empty_like(parts[0][0])
        tp.shard_sum([p[0] for p in parts], out)
        torch.cuda.synchronize()
        assert_bf16_close(f64_host(out), sum(p[1] for p in parts), f"sum of {name}_i")
    if check_unsharded:
        Ao, Bo = bf16_bits_to_f64(inp["A"]), bf16_bits_to_f64(inp["B"])
        out = torch.empty_like(Zs[0][0])
        tp.shard_sum([p[0] for p in Zs], out)
        torch.cuda.synchronize()
        assert_bf16_close(f64_host(out), oracle.mlp_fwd_full(Xo, Ao, Bo, matched=True), "sum of Z_i vs unsharded")


def test_small_mlp_bf16_fwd_bwd_two_shards():
    c = CONFIGS["small_mlp_bf16"]
    _bf16_mlp_case(c["b"] * c["s"], c["h"], c["f_full"], c["N"], c["seed"], c["sigma_w"])


@pytest.mark.parametrize("M,h,f_full,N", [(300, 512, 1536, 2), (257, 384, 1024, 4), (1, 64, 128, 1),
                                          (64, 8, 16, 2)])
def test_ragged_multi_tile(M, h, f_full, N):
    _bf16_mlp_case(M, h, f_full, N, 2000 + M, 0.05)


def test_streamk_epilogues():
    """A shard whose column GEMM, row GEMM, dU and dX products all take the stream-K
    path (16 tiles of 48 k-stages, M = 300, h = f = 1536): the erf-GeLU epilogue (U, Y),
    the float32 one (Z, dX) and the GeLU' one (dU) then run on summed partials in the
    fixup kernel, and every output is compared with the oracle."""
    M, h, f = 300, 1536, 1536
    note(f"bf16 mlp through stream-K M={M} h={h} f={f}")
    fws = tp.mlp_fwd_workspace(M, h, f)
    assert fws > 0, "the column and row GEMMs of this shape should take the stream-K path"
    inp = mlp_inputs(M, h, f, 1, "bf16", 4242, 1.0, 0.05, 1.0)
    A_i, B_i = inp["shards"][0]
    X, dZ, A, B = bf16_dev(inp["X"]), bf16_dev(inp["dZ"]), bf16_dev(A_i), bf16_dev(B_i)
    U, Y, Z = _alloc(M, h, f, torch.bfloat16)
    ws = torch.empty(fws, dtype=torch.uint8, device=DEV)
    tp.mlp_fwd(X, A, B, Y, Z, U_i=U, ws=ws)
    dX, dA, dB, _ = _run_bwd(X, A, B, U, Y, dZ, M, h, f)
    torch.cuda.synchronize()
    Xo, dZo = bf16_bits_to_f64(inp["X"]), bf16_bits_to_f64(inp["dZ"])
    Ao, Bo = bf16_bits_to_f64(A_i), bf16_bits_to_f64(B_i)
    r = oracle.mlp_fwd_shard(Xo, Ao, Bo)
    g = oracle.mlp_bwd_shard(Xo, Ao, Bo, r["U"], r["Y"], dZo)
    for name, got, want in (("U", U, r["U"]), ("Y", Y, r["Y"]), ("Z", Z, r["Z"]), ("dX", dX, g["dX"]),
                            ("dA", dA, g["dA"]), ("dB", dB, g["dB"])):
        assert_bf16_close(f64_host(got), want, name)


def test_empty_batch():
    note("mlp M=0")
    h, f = 64, 128
    X = torch.empty(0, h, dtype=torch.bfloat16, device=DEV)
    A = torch.randn(h, f, device=DEV).to(torch.bfloat16)
    B = torch.randn(f, h, device=DEV).to(torch.bfloat16)
    U, Y, Z = _alloc(0, h, f, torch.bfloat16)
    tp.mlp_fwd(X, A, B, Y, Z, U_i=U)
    dZ = torch.empty(0, h, dtype=torch.bfloat16, device=DEV)
    dX, dA, dB, _ = _run_bwd(X, A, B, U, Y, dZ, 0, h, f)
    torch.cuda.synchronize()
    assert torch.count_nonzero(dA) == 0 and torch.count_nonzero(dB) == 0


def test_column_linear_without_activation():
    note("column_linear bf16 no activation M=130 K=256 N=200")
    rng = np.random.default_rng(5)
    from workloads import bf16_bits
    Xb = bf16_bits(rng.standard_normal((130, 256)).astype(np.float32))
    Wb = bf16_bits((rng.standard_normal((256, 200)) * 0.05).astype(np.float32))
    Y = torch.empty(130, 200, dtype=torch.bfloat16, device=DEV)
    tp.column_linear(bf16_dev(Xb), bf16_dev(Wb), Y, act=None)
    torch.cuda.synchronize()
    from oracle.bf16 import round_to_bf16
    ref = round_to_bf16(bf16_bits_to_f64(Xb) @ bf16_bits_to_f64(Wb))
    assert_bf16_close(f64_host(Y), ref, "X W")


def _gelu_grid():
    """u over [-40, 40] and the small and special values, rounded to bf16 (so that a
    product with one unit weight forms u exactly), padded to a multiple of 8."""
    u = np.concatenate([np.linspace(-40.0, 40.0, 1601), [0.0, -0.0, 1e-3, -1e-3, 0.5, -0.5, 3.5, -3.5, -4.0,
                                                        -6.0, -9.0, -13.0, -88.0, 88.0]])
    u = bf16_bits_to_f64(bf16_bits(u.astype(np.float32)))
    u = np.unique(u)
    pad = -len(u) % 8
    return np.concatenate([u, np.zeros(pad)])


def _gelu_tolerance(u, ref):
    # bf16 rounding of the stored result, plus the epilogue's own error: Phi from the
    # Abramowitz-Stegun 7.1.26 erfc fit in float32 stays within 4e-7 max(1, |u|) of the
    # exact erf form (its bound is absolute: in the far negative tail, where |GeLU| is
    # below ~1e-4, the relative error exceeds bf16 rounding)
    return 2.0 ** -8 * np.abs(ref) + 4e-7 * np.maximum(1.0, np.abs(u))


def test_gelu_epilogue_over_the_range():
    """The column GEMM's GeLU epilogue against the exact erf GeLU, u in [-40, 40]:
    X[:, 0] = u, W[0, :] = 1, every other entry 0, so U = X W = u exactly."""
    u = _gelu_grid()
    M, K, N = len(u), 64, 64
    note(f"GeLU epilogue over {M} values of u")
    X = np.zeros((M, K), np.float32)
    X[:, 0] = u
    W = np.zeros((K, N), np.float32)
    W[0, :] = 1.0
    U = torch.empty(M, N, dtype=torch.bfloat16, device=DEV)
    Y = torch.empty(M, N, dtype=torch.bfloat16, device=DEV)
    tp.column_linear(bf16_dev(bf16_bits(X)), bf16_dev(bf16_bits(W)), Y, U=U, act="gelu")
    torch.cuda.synchronize()
    np.testing.assert_array_equal(f64_host(U), np.repeat(u[:, None], N, axis=1))
    ref = oracle.gelu(u)[:, None]
    err = np.abs(f64_host(Y) - ref)
    tol = _gelu_tolerance(u, oracle.gelu(u))[:, None]
    assert np.all(err <= tol), f"worst u = {u[np.argmax((err / tol).max(axis=1))]}, err/tol = {(err / tol).max():.3f}"


def test_gelu_prime_epilogue_over_the_range():
    """The backward's GeLU' epilogue, dU = (dZ B^T) * GeLU'(U), against the exact form:
    dZ[:, 0] = 1 and B[:, 0] = 1 (else 0) make dZ B^T = 1, and X = I makes dA = X^T dU = dU."""
    u = _gelu_grid()
    h, f = 64, len(u)
    M = h
    note(f"GeLU' epilogue over {f} values of u")
    X = np.eye(M, h, dtype=np.float32)
    Ub = np.repeat(u[None, :], M, axis=0).astype(np.float32)
    dZ = np.zeros((M, h), np.float32)
    dZ[:, 0] = 1.0
    B = np.zeros((f, h), np.float32)
    B[:, 0] = 1.0
    A = np.zeros((h, f), np.float32)
    dX = torch.empty(M, h, dtype=torch.float32, device=DEV)
    dA = torch.empty(h, f, dtype=torch.float32, device=DEV)
    dB = torch.empty(f, h, dtype=torch.float32, device=DEV)
    ws = torch.empty(tp.mlp_bwd_workspace(M, h, f), dtype=torch.uint8, device=DEV)
    tp.mlp_bwd(bf16_dev(bf16_bits(X)), bf16_dev(bf16_bits(A)), bf16_dev(bf16_bits(B)), bf16_dev(bf16_bits(Ub)),
               bf16_dev(bf16_bits(np.zeros((M, f), np.float32))), bf16_dev(bf16_bits(dZ)), dX, dA, dB, ws)
    torch.cuda.synchronize()
    refp = oracle.gelu_prime(u)
    err = np.abs(f64_host(dA) - refp[None, :])
    tol = _gelu_tolerance(u, refp)[None, :]
    assert np.all(err <= tol), f"worst u = {u[np.argmax((err / tol).max(axis=0))]}, err/tol = {(err / tol).max():.3f}"


class TestGpt3MlpShardFullSize:
    """GPT-3-shaped rank shard (M=2048, h=12288, f=6144) in the launch
    configuration the benchmark times; sampled outputs from the oracle."""

    ROWS = np.array([0, 1, 255, 256, 1023, 1500, 2046, 2047])
    COLS = np.array([0, 191, 192, 3000, 6143])

    @pytest.fixture(scope="class")
    def case(self):
        c = CONFIGS["gpt3_mlp_rank_shard"]
        M, h, f = c["b"] * c["s"], c["h"], c["f"]
        inp = mlp_inputs(M, h, f, 1, "bf16", c["seed"], c["sigma_x"], c["sigma_w"], c["sigma_dz"], full=False)
        A_i, B_i = inp["shards"][0]
        note("GPT-3 shard full-size mlp_fwd + mlp_bwd")
        X, A, B, dZ = bf16_dev(inp["X"]), bf16_dev(A_i), bf16_dev(B_i), bf16_dev(inp["dZ"])
        U, Y, Z = _alloc(M, h, f, torch.bfloat16)
        tp.mlp_fwd(X, A, B, Y, Z, U_i=U)
        dX, dA, dB, _ = _run_bwd(X, A, B, U, Y, dZ, M, h, f)
        torch.cuda.synchronize()
        o = dict(X=bf16_bits_to_f64(inp["X"]), A=bf16_bits_to_f64(A_i), B=bf16_bits_to_f64(B_i),
                 dZ=bf16_bits_to_f64(inp["dZ"]))
        g = dict(U=U, Y=Y, Z=Z, dX=dX, dA=dA, dB=dB)
        return o, g

    def test_forward_rows(self, case):
        o, g = case
        r = oracle.mlp_fwd_rows(o["X"], o["A"], o["B"], self.ROWS)
        for k in ("U", "Y", "Z"):
            assert_bf16_close(f64_host(g[k][torch.from_numpy(self.ROWS).to(DEV)]), r[k], f"{k} rows")

    def test_backward_samples(self, case):
        o, g = case
        s = oracle.mlp_bwd_cols(o["X"], o["A"], o["B"], o["dZ"], self.ROWS, self.COLS)
        rows = torch.from_numpy(self.ROWS).to(DEV)
        cols = torch.from_numpy(self.COLS).to(DEV)
        assert_bf16_close(f64_host(g["dA"][:, cols]), s["dA_cols"], "dA columns")
        assert_bf16_close(f64_host(g["dB"][cols, :]), s["dB_rows"], "dB rows")
        assert_bf16_close(f64_host(g["dX"][rows, :]), s["dX_rows"], "dX rows")

    def test_outputs_finite(self, case):
        _, g = case
        for k, t in g.items():
            assert torch.isfinite(t.float()).all(), k

    def test_every_element(self, case):
        """All of U, Y, Z, dX, dA, dB against the float64 oracle over the whole shard."""
        o, g = case
        f = oracle.mlp_fwd_shard(o["X"], o["A"], o["B"])
        for k in ("U", "Y", "Z"):
            assert_bf16_close(f64_host(g[k]), f[k], f"{k} (all elements)")
        b = oracle.mlp_bwd_shard(o["X"], o["A"], o["B"], f["U"], f["Y"], o["dZ"])
        for k in ("dX", "dA", "dB"):
            assert_bf16_close(f64_host(g[k]), b[k], f"{k} (all elements)")


@pytest.mark.parametrize("M,h,f", [(32, 1024, 2048), (300, 512, 768), (1, 64, 128)])
def test_backward_recompute_matches_saved(M, h, f):
    """mlp_bwd without the saved U_i / Y_i recomputes them with the forward's own
    kernel, so every gradient equals the saved-activation run bit for bit."""
    note(f"mlp_bwd recompute vs saved M={M} h={h} f={f}")
    inp = mlp_inputs(M, h, f, 1, "bf16", 4000 + M, 1.0, 0.02, 1.0, full=False)
    A_i, B_i = inp["shards"][0]
    X, A, B, dZ = bf16_dev(inp["X"]), bf16_dev(A_i), bf16_dev(B_i), bf16_dev(inp["dZ"])
    U, Y, Z = _alloc(M, h, f, torch.bfloat16)
    tp.mlp_fwd(X, A, B, Y, Z, U_i=U)
    saved = _run_bwd(X, A, B, U, Y, dZ, M, h, f)[:3]
    ws = torch.empty(tp.mlp_bwd_recompute_workspace(M, h, f), dtype=torch.uint8, device=DEV)
    for U_in, Y_in in ((None, None), (U, None), (None, Y)):
        outs = [torch.full_like(t, float("nan")) for t in saved]
        tp.mlp_bwd(X, A, B, U_in, Y_in, dZ, *outs, ws)
        torch.cuda.synchronize()
        for name, a, b in zip(("dX", "dA", "dB"), outs, saved):
            assert torch.equal(a, b), f"{name} differs (U given: {U_in is not None}, Y given: {Y_in is not None})"


class TestPalmShape:
    """PaLM-shaped rank shard (M = 4096, the page's context; h = 18432, f = 9216):
    forward with saved U, backward with activation recompute; sampled outputs and
    every element against the oracle."""

    ROWS = np.array([0, 255, 256, 1024, 2047, 4095])
    COLS = np.array([0, 191, 192, 5000, 9215])

    @pytest.fixture(scope="class")
    def case(self):
        c = CONFIGS["palm_mlp_rank_shard"]
        M, h, f = c["b"] * c["s"], c["h"], c["f"]
        inp = mlp_inputs(M, h, f, 1, "bf16", c["seed"], c["sigma_x"], c["sigma_w"], c["sigma_dz"], full=False)
        A_i, B_i = inp["shards"][0]
        note("PaLM-shaped mlp_fwd + mlp_bwd with recompute")
        X, A, B, dZ = bf16_dev(inp["X"]), bf16_dev(A_i), bf16_dev(B_i), bf16_dev(inp["dZ"])
        U, Y, Z = _alloc(M, h, f, torch.bfloat16)
        tp.mlp_fwd(X, A, B, Y, Z, U_i=U)
        ws = torch.empty(tp.mlp_bwd_recompute_workspace(M, h, f), dtype=torch.uint8, device=DEV)
        dX = torch.empty(M, h, dtype=torch.float32, device=DEV)
        dA = torch.empty(h, f, dtype=torch.float32, device=DEV)
        dB = torch.empty(f, h, dtype=torch.float32, device=DEV)
        tp.mlp_bwd(X, A, B, None, None, dZ, dX, dA, dB, ws)
        torch.cuda.synchronize()
        o = dict(X=bf16_bits_to_f64(inp["X"]), A=bf16_bits_to_f64(A_i), B=bf16_bits_to_f64(B_i),
                 dZ=bf16_bits_to_f64(inp["dZ"]))
        return o, dict(U=U, Y=Y, Z=Z, dX=dX, dA=dA, dB=dB)

    def test_forward_rows(self, case):
        o, g = case
        r = oracle.mlp_fwd_rows(o["X"], o["A"], o["B"], self.ROWS)
        for k in ("U", "Y", "Z"):
            assert_bf16_close(f64_host(g[k][torch.from_numpy(self.ROWS).to(DEV)]), r[k], f"{k} rows")

    def test_backward_samples(self, case):
        """Sampled dX rows. dA and dB are sums over all 4096 tokens, where a rare bf16
        rounding flip of dU or Y moves a whole column or row: their mean error over
        a few sampled columns is a noisy estimate of the bar's mean over all
        entries, so test_every_element carries the bar for them."""
        o, g = case
        s = oracle.mlp_bwd_cols(o["X"], o["A"], o["B"], o["dZ"], self.ROWS, self.COLS)
        rows = torch.from_numpy(self.ROWS).to(DEV)
        assert_bf16_close(f64_host(g["dX"][rows, :]), s["dX_rows"], "dX rows")

    def test_every_element(self, case):
        """All outputs of the PaLM-shaped shard (backward through recompute)."""
        o, g = case
        f = oracle.mlp_fwd_shard(o["X"], o["A"], o["B"])
        for k in ("U", "Y", "Z"):
            assert_bf16_close(f64_host(g[k]), f[k], f"{k} (all elements)")
        b = oracle.mlp_bwd_shard(o["X"], o["A"], o["B"], f["U"], f["Y"], o["dZ"])
        for k in ("dX", "dA", "dB"):
            assert_bf16_close(f64_host(g[k]), b[k], f"{k} (all elements)")

    def test_outputs_finite(self, case):
        _, g = case
        for k, t in g.items():
            assert torch.isfinite(t.float()).all(), k
