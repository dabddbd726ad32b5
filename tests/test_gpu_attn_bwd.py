"""GPU parity of the attention backward (core and whole shard) against the
float64 oracle, through the C ABI.

Tolerance: the bf16 bar of every other product, normwise max|g - r| / max|r|
<= 2e-2 and mean|g - r| <= 1e-3, against the oracle in matched mode (bf16
storage of Q, K, V, O, dO and dQKV where the GPU stores them). The kernels feed
P and dS to the MFMAs as hi/lo bf16 pairs (and the training forward feeds P to
P V that way), so the stored bf16 values round as the exact ones do in all but
a small fraction of entries; the weight gradients dWo = O^T dOut and
dWqkv = X^T dQKV, sums over every token, then stay within the bar. The
log-sum-exp is float32 throughout: |g - r| <= 1e-4.
"""
import numpy as np
import pytest
import torch

import oracle
from oracle.bf16 import bf16_bits_to_f64
from tests.gpu_util import DEV, assert_bf16_close, bf16_dev, f64_host, note
from workloads import CONFIGS, attn_inputs, bf16_bits, draw_normal_f32

pytestmark = pytest.mark.gpu

tp = pytest.importorskip("attention_shard_math_amd")


def assert_grad_close(g, r, what):
    assert_bf16_close(g, r, what)


def _core_case(b, s, Hl, d, causal, seed):
    rng = np.random.default_rng(seed)
    w = Hl * d
    qkv = bf16_bits(draw_normal_f32(rng, (b * s, 3 * w), 1.0))
    dO = bf16_bits(draw_normal_f32(rng, (b * s, w), 1.0))
    Q = bf16_dev(qkv)
    O = torch.empty(b * s, w, dtype=torch.bfloat16, device=DEV)
    lse = torch.full((b, Hl, s), float("nan"), dtype=torch.float32, device=DEV)
    tp.attn_core_train(Q, O, lse, b, s, Hl, d, causal)
    dq = torch.full((b * s, 3 * w), float("nan"), dtype=torch.bfloat16, device=DEV)
    ws = torch.empty(tp.attn_core_bwd_workspace(b, s, Hl, d), dtype=torch.uint8, device=DEV)
    tp.attn_core_bwd(Q, O, bf16_dev(dO), lse, dq, ws, b, s, Hl, d, causal)
    return qkv, dO, O, lse, dq, (Q, bf16_dev(dO), ws)


# Walks longer than 16 key (or query) tiles of 32 are cut into chunks whose fp32
# partials a combine pass adds: s = 513 and 530 (causal) and s = 600 (every block,
# not causal) cover that path for both head sizes. d = 384 (blocks of 64 rows, a
# step's work split over four waves): ragged lengths (301, 200, 1, 8), chunked walks
# (700 causal, 530 not), and blocks whose second half lies past the end.
@pytest.mark.parametrize("b,s,Hl,d,causal", [(2, 300, 2, 128, True), (1, 77, 3, 64, True),
                                              (2, 200, 2, 128, False), (1, 1, 1, 128, True),
                                              (3, 129, 1, 64, False), (1, 513, 1, 128, True),
                                              (2, 530, 1, 64, True), (1, 600, 2, 64, False),
                                              (1, 304, 2, 384, True), (2, 200, 1, 384, False),
                                              (1, 8, 1, 384, True), (1, 301, 2, 384, True),
                                              (1, 1, 1, 384, True), (1, 700, 1, 384, True),
                                              (2, 530, 1, 384, False), (1, 100, 1, 384, True),
                                              (2, 150, 2, 384, True)])
def test_core_backward(b, s, Hl, d, causal):
    note(f"attn_core_bwd b={b} s={s} Hl={Hl} d={d} causal={causal}")
    qkv, dO, O, lse, dq, _ = _core_case(b, s, Hl, d, causal, 90 + s + d)
    torch.cuda.synchronize()
    q = bf16_bits_to_f64(qkv)
    w = Hl * d
    Qo, Ko, Vo = q[:, :w], q[:, w:2 * w], q[:, 2 * w:]
    np.testing.assert_allclose(f64_host(lse), oracle.attn_lse(Qo, Ko, b, s, Hl, d, causal), rtol=0, atol=1e-4)
    rq, rk, rv = oracle.attn_core_bwd(Qo, Ko, Vo, bf16_bits_to_f64(dO), b, s, Hl, d, causal)
    g = f64_host(dq)
    assert_grad_close(g[:, :w], rq, "dQ")
    assert_grad_close(g[:, w:2 * w], rk, "dK")
    assert_grad_close(g[:, 2 * w:], rv, "dV")


@pytest.mark.parametrize("Hl,d", [(2, 128), (1, 384)])
def test_core_backward_is_deterministic(Hl, d):
    b, s = 1, 700
    note(f"attn_core_bwd twice, bit-identical, d={d}")
    qkv, dO, O, lse, dq, (Q, dOd, ws) = _core_case(b, s, Hl, d, True, 99)
    dq2 = torch.empty_like(dq)
    tp.attn_core_bwd(Q, O, dOd, lse, dq2, ws, b, s, Hl, d, True)
    torch.cuda.synchronize()
    assert torch.equal(dq.view(torch.int16), dq2.view(torch.int16))


def _shard_case(b, s, h, Hl, d, ai, dOut_bits, causal=True):
    w = Hl * d
    X, Wqkv, Wo = (bf16_dev(ai[k]) for k in ("X", "Wqkv", "Wo"))
    out = torch.empty(b * s, h, dtype=torch.float32, device=DEV)
    QKV = torch.empty(b * s, 3 * w, dtype=torch.bfloat16, device=DEV)
    O = torch.empty(b * s, w, dtype=torch.bfloat16, device=DEV)
    lse = torch.empty(b, Hl, s, dtype=torch.float32, device=DEV)
    tp.attn_fwd_train(X, Wqkv, Wo, out, QKV, O, lse, b, s, Hl, d, causal)
    dX = torch.full((b * s, h), float("nan"), dtype=torch.float32, device=DEV)
    dWqkv = torch.full((h, 3 * w), float("nan"), dtype=torch.float32, device=DEV)
    dWo = torch.full((w, h), float("nan"), dtype=torch.float32, device=DEV)
    ws = torch.empty(tp.attn_bwd_workspace(b, s, h, Hl, d), dtype=torch.uint8, device=DEV)
    tp.attn_bwd(X, Wqkv, Wo, QKV, O, lse, bf16_dev(dOut_bits), dX, dWqkv, dWo, ws, b, s, Hl, d, causal)
    return out, dX, dWqkv, dWo, ws


# Small and ragged shards drawn with the GPT-3 shard's activation statistics: the
# weights' sigma is 0.006 * sqrt(12288 / h), so that Q, K, V, O and the gradients
# have the scale they have at h = 12288 (the mean-abs bar is absolute).
# 384-wide heads use the PaLM shard's scale, 0.005 * sqrt(18432 / h).
@pytest.mark.parametrize("b,s,h,Hl,d", [(2, 300, 512, 2, 128), (1, 150, 256, 4, 64), (1, 264, 768, 2, 384)])
def test_shard_backward(b, s, h, Hl, d):
    note(f"attn_fwd_train + attn_bwd b={b} s={s} h={h} Hl={Hl} d={d}")
    sigma_w = 0.005 * np.sqrt(18432 / h) if d == 384 else 0.006 * np.sqrt(12288 / h)
    ai = attn_inputs(b, s, h, Hl, d, 180 + s, 1.0, sigma_w)
    dOut = bf16_bits(draw_normal_f32(np.random.default_rng(181 + s), (b * s, h), 1.0))
    out, dX, dWqkv, dWo, ws = _shard_case(b, s, h, Hl, d, ai, dOut)
    torch.cuda.synchronize()
    r = oracle.attn_shard_bwd(*(bf16_bits_to_f64(ai[k]) for k in ("X", "Wqkv", "Wo")), bf16_bits_to_f64(dOut),
                              b, s, Hl, d, True, matched=True)
    assert_grad_close(f64_host(out), r["fwd"]["out"], "out_partial")
    assert_grad_close(f64_host(dWo), r["dWo"], "dWo_i")
    assert_grad_close(f64_host(dWqkv), r["dWqkv"], "dWqkv_i")
    assert_grad_close(f64_host(dX), r["dX"], "dX_i")
    w = Hl * d
    dO = ws[:b * s * w * 2].view(torch.bfloat16).view(b * s, w)
    assert_grad_close(f64_host(dO), r["dO"], "dO")


@pytest.mark.parametrize("cfg", ["gpt3_attn_rank_shard", "palm_attn_rank_shard"])
def test_full_size_shard_backward(cfg):
    """GPT-3 shard (12 local heads of 128, s = 2048, h = 12288) and PaLM shard (6
    local heads of 384, s = 4096, h = 18432): every output against the full
    float64 oracle."""
    c = CONFIGS[cfg]
    b, s, h, d = c["b"], c["s"], c["h"], c["d_head"]
    Hl = c["n_heads"] // c["N"]
    ai = attn_inputs(b, s, h, Hl, d, c["seed"], c["sigma_x"], c["sigma_w"])
    dOut = bf16_bits(draw_normal_f32(np.random.default_rng(c["seed"] + 1), (b * s, h), 1.0))
    note(f"attn_fwd_train + attn_bwd {cfg} full size")
    out, dX, dWqkv, dWo, ws = _shard_case(b, s, h, Hl, d, ai, dOut)
    torch.cuda.synchronize()
    r = oracle.attn_shard_bwd(*(bf16_bits_to_f64(ai[k]) for k in ("X", "Wqkv", "Wo")), bf16_bits_to_f64(dOut),
                              b, s, Hl, d, True, matched=True)
    assert_grad_close(f64_host(out), r["fwd"]["out"], "out_partial (all elements)")
    assert_grad_close(f64_host(dWo), r["dWo"], "dWo_i")
    assert_grad_close(f64_host(dWqkv), r["dWqkv"], "dWqkv_i")
    assert_grad_close(f64_host(dX), r["dX"], "dX_i")
    w = Hl * d
    off = -(-b * s * w * 2 // 256) * 256
    dqkv = ws[off:off + b * s * 3 * w * 2].view(torch.bfloat16).view(b * s, 3 * w)
    assert_grad_close(f64_host(dqkv), r["dQKV"], "dQKV")
