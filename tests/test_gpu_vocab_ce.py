"""GPU parity of the vocabulary-parallel output layer and cross-entropy against
the float64 oracle, through the C ABI.

The GPU carries each rank's row sum of exp relative to its row maximum
(rowmax_i, sumexp_i = sum exp(logit - rowmax_i)); the page's sum of exp is
exp(rowmax_i) * sumexp_i, so the rank's log-sum-exp rowmax_i + log(sumexp_i) is
compared with the log of the oracle's plain float64 sum.

Tolerance: the inputs are bf16 and used exactly by both sides, and the GPU keeps
every intermediate in float32 (logits accumulated over h terms, exp, the row
sums, the rank sums, log). The expected error of a logit is about
u32 * sqrt(h/2) of its row's scale (u32 = 2^-24, so ~5e-6 at h = 12288, logit
sigma ~2.2); the bounds below leave a factor of >= 10: row maxima and
target logits 1e-4 absolute, the per-rank log-sum-exp 1e-4 absolute (a 1e-4
relative bound on the sum of exp), row losses 2e-4 absolute, the scalar loss
1e-5 relative.
"""
import numpy as np
import pytest
import torch

import oracle
from oracle.bf16 import bf16_bits_to_f64
from tests.gpu_util import DEV, bf16_dev, f64_host, note
from workloads import CONFIGS, ce_inputs

pytestmark = pytest.mark.gpu

tp = pytest.importorskip("attention_shard_math_amd")

LOGIT_ATOL = 1e-4
LSE_ATOL = 1e-4
LOSS_ATOL = 2e-4
LOSS_SUM_RTOL = 1e-5


def _rank(Hd, Ed_i, td, lo, hi):
    M, h = Hd.shape
    m = torch.full((M,), float("nan"), dtype=torch.float32, device=DEV)
    s = torch.full((M,), float("nan"), dtype=torch.float32, device=DEV)
    t = torch.full((M,), float("nan"), dtype=torch.float32, device=DEV)
    ws = torch.empty(max(tp.vocab_ce_workspace(M, h, lo, hi), 1), dtype=torch.uint8, device=DEV)
    tp.vocab_ce_partials(Hd, Ed_i, td, lo, hi, m, s, t, ws)
    return m, s, t, ws


def _combine(ms, ss, ts):
    M = ss[0].numel()
    rows = torch.full((M,), float("nan"), dtype=torch.float32, device=DEV)
    tot = torch.full((1,), float("nan"), dtype=torch.float32, device=DEV)
    tp.vocab_ce_loss(ms, ss, ts, rows, tot)
    return rows, tot


def _assert_lse(m, s, sumexp_ref, what):
    g = f64_host(m) + np.log(f64_host(s))
    np.testing.assert_allclose(g, np.log(sumexp_ref), rtol=0, atol=LSE_ATOL, err_msg=what)


# The logits GEMM reduces each 96-column block of a row in its epilogue. The cases
# cover a slice ending inside a block (520 = 5 * 96 + 40), blocks wholly past the
# slice's end (264 and 8 columns), stream-K with every tile split (37 x 520), and
# 256 tiles that fill the grid (2048 x 6144: the tile kernel, no stream-K).
@pytest.mark.parametrize("M,h,v,N", [(300, 328, 2080, 4), (37, 64, 520, 1), (1, 8, 64, 8), (515, 256, 1536, 16),
                                     (100, 64, 528, 2), (2048, 64, 6144, 1)])
def test_small_against_oracle(M, h, v, N):
    inp = ce_inputs(M, h, v, seed=4242 + M, sigma_h=1.0, sigma_w=0.3)
    t = inp["targets"].copy()
    # targets on both edges of the slices as well as uniform ones
    w = v // N
    for k in range(min(M, 2 * N)):
        t[k] = (k // 2) * w + (0 if k % 2 == 0 else w - 1)
    Ho, Eo = bf16_bits_to_f64(inp["H"]), bf16_bits_to_f64(inp["E"])
    Hd, Ed, td = bf16_dev(inp["H"]), bf16_dev(inp["E"]), torch.from_numpy(t).to(DEV)
    ms, ss, ts, refs = [], [], [], []
    for i in range(N):
        lo, hi = i * w, (i + 1) * w
        note(f"vocab_ce_partials M={M} h={h} slice [{lo},{hi}) of {v}")
        m, s, tl, _ = _rank(Hd, Ed[lo:hi], td, lo, hi)
        torch.cuda.synchronize()
        r = oracle.vocab_ce_partials(Ho, Eo[lo:hi], t, lo, hi)
        np.testing.assert_allclose(f64_host(m), r["logits"].max(axis=1), rtol=0, atol=LOGIT_ATOL)
        _assert_lse(m, s, r["sumexp"], "rank log-sum-exp")
        np.testing.assert_allclose(f64_host(tl), r["tlogit"], rtol=0, atol=LOGIT_ATOL)
        # rows whose target lies outside the slice carry exactly 0
        miss = (t < lo) | (t >= hi)
        assert np.all(f64_host(tl)[miss] == 0.0)
        ms.append(m)
        ss.append(s)
        ts.append(tl)
        refs.append(r)
    note(f"vocab_ce_loss M={M} parts={N}")
    rows, tot = _combine(ms, ss, ts)
    torch.cuda.synchronize()
    want = oracle.vocab_ce_combine([r["sumexp"] for r in refs], [r["tlogit"] for r in refs])
    np.testing.assert_allclose(f64_host(rows), want["loss_rows"], rtol=0, atol=LOSS_ATOL)
    assert abs(float(tot.item()) - want["loss"]) <= LOSS_SUM_RTOL * abs(want["loss"]) + LOSS_ATOL
    # and the same loss as the unsharded definition over the whole vocabulary
    whole = oracle.vocab_ce_sharded(Ho, Eo, t, 1)
    np.testing.assert_allclose(f64_host(rows), whole["loss_rows"], rtol=0, atol=LOSS_ATOL)


def test_empty_rows():
    note("vocab_ce empty M=0")
    Hd = torch.empty(0, 64, dtype=torch.bfloat16, device=DEV)
    Ed = torch.zeros(64, 64, dtype=torch.bfloat16, device=DEV)
    td = torch.empty(0, dtype=torch.int32, device=DEV)
    s = torch.empty(0, dtype=torch.float32, device=DEV)
    tp.vocab_ce_partials(Hd, Ed, td, 0, 64, s, s.clone(), s.clone(), None)
    rows = torch.empty(0, dtype=torch.float32, device=DEV)
    tot = torch.full((1,), float("nan"), dtype=torch.float32, device=DEV)
    tp.vocab_ce_loss([s, s], [s, s], [s, s], rows, tot)
    torch.cuda.synchronize()
    assert float(tot.item()) == 0.0


def test_zero_table_gives_log_v():
    """With E = 0 every logit is 0, so every row's loss is log v exactly as in
    float64 up to float32 rounding of log."""
    M, h, v, N = 70, 64, 1024, 8
    note("vocab_ce zero table")
    Hd = torch.randn(M, h, device=DEV).to(torch.bfloat16)
    Ed = torch.zeros(v, h, dtype=torch.bfloat16, device=DEV)
    td = torch.randint(0, v, (M,), dtype=torch.int32, device=DEV)
    w = v // N
    ms, ss, ts = [], [], []
    for i in range(N):
        m, s, t, _ = _rank(Hd, Ed[i * w:(i + 1) * w], td, i * w, (i + 1) * w)
        ms.append(m)
        ss.append(s)
        ts.append(t)
    rows, tot = _combine(ms, ss, ts)
    torch.cuda.synchronize()
    np.testing.assert_allclose(f64_host(rows), np.full(M, np.log(v)), rtol=1e-6)
    for m, s in zip(ms, ss):
        assert np.all(f64_host(m) == 0.0)
        assert np.all(f64_host(s) == w)


@pytest.mark.parametrize("M,h,v,N", [(96, 64, 1024, 4), (40, 256, 2112, 8)])
def test_large_logits_do_not_overflow(M, h, v, N):
    """Logits far above 88.7 (where exp overflows float32): each rank's sum is
    carried relative to its row maximum, so the losses stay finite and match the
    float64 oracle, which forms exp(logit) itself."""
    inp = ce_inputs(M, h, v, seed=77 + M, sigma_h=1.0, sigma_w=60.0 / np.sqrt(h))
    t = inp["targets"]
    Ho, Eo = bf16_bits_to_f64(inp["H"]), bf16_bits_to_f64(inp["E"])
    assert (Ho @ Eo.T).max() > 100.0
    Hd, Ed, td = bf16_dev(inp["H"]), bf16_dev(inp["E"]), torch.from_numpy(t).to(DEV)
    w = v // N
    ms, ss, ts, refs = [], [], [], []
    for i in range(N):
        lo, hi = i * w, (i + 1) * w
        note(f"vocab_ce_partials large logits M={M} h={h} slice [{lo},{hi})")
        m, s, tl, _ = _rank(Hd, Ed[lo:hi], td, lo, hi)
        ms.append(m)
        ss.append(s)
        ts.append(tl)
        refs.append(oracle.vocab_ce_partials(Ho, Eo[lo:hi], t, lo, hi))
    rows, tot = _combine(ms, ss, ts)
    torch.cuda.synchronize()
    for i in range(N):
        # the logits reach ~200: their float32 rounding is 2^-17 absolute
        np.testing.assert_allclose(f64_host(ms[i]), refs[i]["logits"].max(axis=1), rtol=0, atol=1e-3)
        g = f64_host(ms[i]) + np.log(f64_host(ss[i]))
        np.testing.assert_allclose(g, np.log(refs[i]["sumexp"]), rtol=0, atol=1e-3)
    want = oracle.vocab_ce_combine([r["sumexp"] for r in refs], [r["tlogit"] for r in refs])
    g_rows = f64_host(rows)
    assert np.all(np.isfinite(g_rows))
    np.testing.assert_allclose(g_rows, want["loss_rows"], rtol=0, atol=2e-3)


def test_full_size_sampled_rows():
    """GPT-3 vocabulary (50304 = 8 x 6288), h = 12288, 2048 rows, all eight
    slices run on the GPU; the oracle recomputes sampled rows' partial sums, then
    every row's partial sums and loss over the whole vocabulary."""
    c = CONFIGS["vocab_parallel_ce"]
    M, h, v, N = c["b"] * c["s"], c["h"], c["v"], c["N"]
    inp = ce_inputs(M, h, v, c["seed"], c["sigma_h"], c["sigma_w"])
    t = inp["targets"]
    Hd, Ed, td = bf16_dev(inp["H"]), bf16_dev(inp["E"]), torch.from_numpy(t).to(DEV)
    w = v // N
    ms, ss, ts = [], [], []
    rows_s = np.array([0, 1, 777, 1500, M - 2, M - 1])
    rows_d = torch.from_numpy(rows_s).to(DEV)
    for i in range(N):
        note(f"vocab_ce_partials full size slice {i}/{N}")
        m, s, tl, _ = _rank(Hd, Ed[i * w:(i + 1) * w], td, i * w, (i + 1) * w)
        ms.append(m)
        ss.append(s)
        ts.append(tl)
    note("vocab_ce_loss full size")
    rows, tot = _combine(ms, ss, ts)
    torch.cuda.synchronize()
    Ho = bf16_bits_to_f64(inp["H"][rows_s])
    refs = [oracle.vocab_ce_partials(Ho, bf16_bits_to_f64(inp["E"][i * w:(i + 1) * w]), t[rows_s], i * w,
                                     (i + 1) * w) for i in range(N)]
    for i in range(N):
        np.testing.assert_allclose(f64_host(ms[i])[rows_s], refs[i]["logits"].max(axis=1), rtol=0,
                                   atol=LOGIT_ATOL)
        _assert_lse(ms[i][rows_d], ss[i][rows_d], refs[i]["sumexp"], "sampled rows' log-sum-exp")
        np.testing.assert_allclose(f64_host(ts[i])[rows_s], refs[i]["tlogit"], rtol=0, atol=LOGIT_ATOL)
    want = oracle.vocab_ce_combine([r["sumexp"] for r in refs], [r["tlogit"] for r in refs])
    g_rows = f64_host(rows)
    np.testing.assert_allclose(g_rows[rows_s], want["loss_rows"], rtol=0, atol=LOSS_ATOL)
    assert np.all(np.isfinite(g_rows))
    # each target is held by exactly one slice: the rank sum of the target logits
    # equals the one nonzero term
    held = np.stack([f64_host(x) for x in ts])
    assert np.all((held != 0).sum(axis=0) <= 1)
    assert abs(float(tot.item()) - g_rows.sum()) <= LOSS_SUM_RTOL * abs(g_rows.sum())
    # every row: the oracle over the whole vocabulary, slice by slice
    Hall = bf16_bits_to_f64(inp["H"])
    full = [oracle.vocab_ce_partials(Hall, bf16_bits_to_f64(inp["E"][i * w:(i + 1) * w]), t, i * w, (i + 1) * w)
            for i in range(N)]
    for i in range(N):
        _assert_lse(ms[i], ss[i], full[i]["sumexp"], "every row's log-sum-exp")
        np.testing.assert_allclose(f64_host(ts[i]), full[i]["tlogit"], rtol=0, atol=LOGIT_ATOL)
    want_all = oracle.vocab_ce_combine([x["sumexp"] for x in full], [x["tlogit"] for x in full])
    np.testing.assert_allclose(g_rows, want_all["loss_rows"], rtol=0, atol=LOSS_ATOL)
    assert abs(float(tot.item()) - want_all["loss"]) <= LOSS_SUM_RTOL * abs(want_all["loss"])
