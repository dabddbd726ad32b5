"""GPU parity of the attention shard (QKV GEMM, fused causal attention, row-
parallel output projection) against the float64 oracle."""
import numpy as np
import pytest
import torch

import oracle
from oracle.bf16 import bf16_bits_to_f64
from tests.gpu_util import DEV, assert_bf16_close, bf16_dev, f64_host, note
from workloads import CONFIGS, attn_inputs, bf16_bits, draw_normal_f32

pytestmark = pytest.mark.gpu

tp = pytest.importorskip("attention_shard_math_amd")


@pytest.mark.parametrize("b,s,Hl,d,causal", [(2, 300, 2, 128, True), (1, 77, 3, 64, True),
                                              (2, 200, 2, 128, False), (1, 1, 1, 128, True),
                                              (3, 129, 1, 64, False), (1, 300, 2, 384, True),
                                              (2, 200, 1, 384, False), (1, 1, 1, 384, True)])
def test_attn_core(b, s, Hl, d, causal):
    note(f"attn_core b={b} s={s} Hl={Hl} d={d} causal={causal}")
    rng = np.random.default_rng(71 + s)
    qkv = bf16_bits(draw_normal_f32(rng, (b * s, 3 * Hl * d), 1.0))
    O = torch.empty(b * s, Hl * d, dtype=torch.bfloat16, device=DEV)
    tp.attn_core(bf16_dev(qkv), O, b, s, Hl, d, causal)
    torch.cuda.synchronize()
    q = bf16_bits_to_f64(qkv)
    w = Hl * d
    ref = oracle.attn_core(q[:, :w], q[:, w:2 * w], q[:, 2 * w:], b, s, Hl, d, causal)
    assert_bf16_close(f64_host(O), ref, "O")


# The kernels keep a ring of 64-key stages of K and V in LDS (four stages for
# d <= 128, two for d = 384): sequences of one to five stages, and lengths one key
# past a stage boundary, exercise every start-up, wrap and drain path of that ring.
@pytest.mark.parametrize("s", [63, 64, 65, 128, 129, 192, 193, 256, 257])
@pytest.mark.parametrize("d,causal", [(128, True), (128, False), (64, True), (384, True), (384, False)])
def test_attn_core_stage_counts(s, d, causal):
    note(f"attn_core stages s={s} d={d} causal={causal}")
    b, Hl = 1, 2
    rng = np.random.default_rng(500 + s + d)
    qkv = bf16_bits(draw_normal_f32(rng, (b * s, 3 * Hl * d), 1.0))
    O = torch.empty(b * s, Hl * d, dtype=torch.bfloat16, device=DEV)
    tp.attn_core(bf16_dev(qkv), O, b, s, Hl, d, causal)
    torch.cuda.synchronize()
    q = bf16_bits_to_f64(qkv)
    w = Hl * d
    ref = oracle.attn_core(q[:, :w], q[:, w:2 * w], q[:, 2 * w:], b, s, Hl, d, causal)
    assert_bf16_close(f64_host(O), ref, "O")


# The training variant (P as a hi/lo bf16 pair, and the log-sum-exp written for the
# backward) over the same ring paths, including the wrap of the four-stage ring.
@pytest.mark.parametrize("s", [64, 65, 192, 257, 320, 321])
@pytest.mark.parametrize("d,causal", [(128, True), (128, False), (64, False), (384, True)])
def test_attn_core_train_stage_counts(s, d, causal):
    note(f"attn_core_train stages s={s} d={d} causal={causal}")
    b, Hl = 1, 2
    rng = np.random.default_rng(900 + s + d)
    qkv = bf16_bits(draw_normal_f32(rng, (b * s, 3 * Hl * d), 1.0))
    O = torch.empty(b * s, Hl * d, dtype=torch.bfloat16, device=DEV)
    lse = torch.full((b, Hl, s), float("nan"), dtype=torch.float32, device=DEV)
    tp.attn_core_train(bf16_dev(qkv), O, lse, b, s, Hl, d, causal)
    torch.cuda.synchronize()
    q = bf16_bits_to_f64(qkv)
    w = Hl * d
    ref = oracle.attn_core(q[:, :w], q[:, w:2 * w], q[:, 2 * w:], b, s, Hl, d, causal)
    assert_bf16_close(f64_host(O), ref, "O")
    ref_lse = oracle.attn_lse(q[:, :w], q[:, w:2 * w], b, s, Hl, d, causal)
    np.testing.assert_allclose(f64_host(lse), ref_lse, rtol=0, atol=1e-4)


# Ragged lengths of one to sixteen 64-key stages per query block, d = 64 and 128.
@pytest.mark.parametrize("b,s,h,Hl,d", [(2, 300, 512, 2, 128), (1, 150, 256, 4, 64), (1, 1000, 256, 2, 128),
                                        (2, 700, 256, 2, 64), (1, 600, 768, 2, 384), (2, 130, 384, 1, 384)])
def test_attn_fwd_ragged(b, s, h, Hl, d):
    note(f"attn_fwd b={b} s={s} h={h} Hl={Hl} d={d}")
    ai = attn_inputs(b, s, h, Hl, d, 80 + s, 1.0, 0.05)
    out = torch.empty(b * s, h, dtype=torch.float32, device=DEV)
    ws = torch.empty(tp.attn_fwd_workspace(b, s, Hl, d, h=h), dtype=torch.uint8, device=DEV)
    tp.attn_fwd(*(bf16_dev(ai[k]) for k in ("X", "Wqkv", "Wo")), out, ws, b, s, Hl, d, True)
    torch.cuda.synchronize()
    r = oracle.attn_shard(*(bf16_bits_to_f64(ai[k]) for k in ("X", "Wqkv", "Wo")), b, s, Hl, d)
    assert_bf16_close(f64_host(out), r["out"], "out_partial")
    qkv = ws[: b * s * 3 * Hl * d * 2].view(torch.bfloat16).view(b * s, 3 * Hl * d)
    w = Hl * d
    assert_bf16_close(f64_host(qkv[:, :w]), r["Q"], "Q")
    assert_bf16_close(f64_host(qkv[:, 2 * w:]), r["V"], "V")
    o_off = (b * s * 3 * w * 2 + 255) // 256 * 256
    O = ws[o_off: o_off + b * s * w * 2].view(torch.bfloat16).view(b * s, w)
    assert_bf16_close(f64_host(O), r["O"], "O")


def test_gpt3_attn_shard_full_size_sampled_rows():
    c = CONFIGS["gpt3_attn_rank_shard"]
    b, s, h, d = c["b"], c["s"], c["h"], c["d_head"]
    Hl = c["n_heads"] // c["N"]
    ai = attn_inputs(b, s, h, Hl, d, c["seed"], c["sigma_x"], c["sigma_w"])
    note("attn_fwd GPT-3 shard full size")
    out = torch.empty(b * s, h, dtype=torch.float32, device=DEV)
    ws = torch.empty(tp.attn_fwd_workspace(b, s, Hl, d, h=h), dtype=torch.uint8, device=DEV)
    tp.attn_fwd(*(bf16_dev(ai[k]) for k in ("X", "Wqkv", "Wo")), out, ws, b, s, Hl, d, True)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all()
    rows = np.array([0, 1, 63, 64, 127, 128, 1000, 1024, 1500, 2047])
    r = oracle.attn_shard_rows(*(bf16_bits_to_f64(ai[k]) for k in ("X", "Wqkv", "Wo")), b, s, Hl, d, rows)
    assert_bf16_close(f64_host(out[torch.from_numpy(rows).to(DEV)]), r["out"], "out rows")
    w = Hl * d
    o_off = (b * s * 3 * w * 2 + 255) // 256 * 256
    O = ws[o_off: o_off + b * s * w * 2].view(torch.bfloat16).view(b * s, w)
    assert_bf16_close(f64_host(O[torch.from_numpy(rows).to(DEV)]), r["O"], "O rows")


def test_gpt3_attn_shard_full_size_every_element():
    """The call the benchmark times (tp_attn_fwd at the GPT-3 shard, 12 local heads
    of 128, s = 2048, h = 12288): every element of Q, K, V, O and out_partial
    against the float64 oracle in matched mode."""
    c = CONFIGS["gpt3_attn_rank_shard"]
    b, s, h, d = c["b"], c["s"], c["h"], c["d_head"]
    Hl = c["n_heads"] // c["N"]
    ai = attn_inputs(b, s, h, Hl, d, c["seed"], c["sigma_x"], c["sigma_w"])
    note("attn_fwd GPT-3 shard full size, every element")
    out = torch.full((b * s, h), float("nan"), dtype=torch.float32, device=DEV)
    ws = torch.empty(tp.attn_fwd_workspace(b, s, Hl, d, h=h), dtype=torch.uint8, device=DEV)
    tp.attn_fwd(*(bf16_dev(ai[k]) for k in ("X", "Wqkv", "Wo")), out, ws, b, s, Hl, d, True)
    torch.cuda.synchronize()
    r = oracle.attn_shard(*(bf16_bits_to_f64(ai[k]) for k in ("X", "Wqkv", "Wo")), b, s, Hl, d)
    w = Hl * d
    qkv = f64_host(ws[: b * s * 3 * w * 2].view(torch.bfloat16).view(b * s, 3 * w))
    assert_bf16_close(qkv[:, :w], r["Q"], "Q (all elements)")
    assert_bf16_close(qkv[:, w:2 * w], r["K"], "K (all elements)")
    assert_bf16_close(qkv[:, 2 * w:], r["V"], "V (all elements)")
    o_off = (b * s * 3 * w * 2 + 255) // 256 * 256
    O = ws[o_off: o_off + b * s * w * 2].view(torch.bfloat16).view(b * s, w)
    assert_bf16_close(f64_host(O), r["O"], "O (all elements)")
    assert_bf16_close(f64_host(out), r["out"], "out_partial (all elements)")


def test_palm_attn_shard_full_size_every_element():
    """PaLM 540B shard: 48 heads of 384 over 8 ranks (6 local heads), context 4096,
    h = 18432: every element of Q, K, V, O and out_partial of tp_attn_fwd."""
    c = CONFIGS["palm_attn_rank_shard"]
    b, s, h, d = c["b"], c["s"], c["h"], c["d_head"]
    Hl = c["n_heads"] // c["N"]
    ai = attn_inputs(b, s, h, Hl, d, c["seed"], c["sigma_x"], c["sigma_w"])
    note("attn_fwd PaLM shard full size, every element")
    out = torch.full((b * s, h), float("nan"), dtype=torch.float32, device=DEV)
    ws = torch.empty(tp.attn_fwd_workspace(b, s, Hl, d, h=h), dtype=torch.uint8, device=DEV)
    tp.attn_fwd(*(bf16_dev(ai[k]) for k in ("X", "Wqkv", "Wo")), out, ws, b, s, Hl, d, True)
    torch.cuda.synchronize()
    r = oracle.attn_shard(*(bf16_bits_to_f64(ai[k]) for k in ("X", "Wqkv", "Wo")), b, s, Hl, d)
    w = Hl * d
    qkv = f64_host(ws[: b * s * 3 * w * 2].view(torch.bfloat16).view(b * s, 3 * w))
    for i, k in enumerate("QKV"):
        assert_bf16_close(qkv[:, i * w:(i + 1) * w], r[k], f"{k} (all elements)")
    o_off = (b * s * 3 * w * 2 + 255) // 256 * 256
    O = ws[o_off: o_off + b * s * w * 2].view(torch.bfloat16).view(b * s, w)
    assert_bf16_close(f64_host(O), r["O"], "O (all elements)")
    assert_bf16_close(f64_host(out), r["out"], "out_partial (all elements)")
