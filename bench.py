"""Benchmark of one tensor-parallel rank's hot path on one MI355X.

A step is one pass of every step of the rank-shard path over one batch of
synthetic input already resident in HBM:
  MLP forward      column GEMM + erf-GeLU, row GEMM -> fp32 partial
                   (GPT-3 175B shard: X [2048, 12288], A_i [12288, 6144], B_i [6144, 12288])
  MLP backward     dU, dB_i, dA_i, dX_i
  shard-sum        8 fp32 partials [2048, 12288] summed in fixed order (all-reduce stand-in)
  attention shard  QKV GEMM, fused causal attention over 12 local heads of 128,
                   row-parallel Wo GEMM -> fp32 partial
  vocab gather     one rank's shard (6288 rows of 12288) for 8 x 2048 token ids

The reported value is the metric: TFLOP/s of the MLP forward + backward
(1855.43 GFLOP per step), timed with HIP events on the launch stream over the
timed steps. ms_per_step is the wall time of whole steps. Per-row times (mean,
median, min and p90 over the timed steps) and roofline fractions (on the mean) are
in "breakdown"; "roofline" is for the dominant kernel.
Prints one JSON line.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6   # MI355X dense bf16 MFMA (256 CU x 2.4 GHz x 4096 flop/clk)
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
METRIC = "TFLOP/s and % bf16 MFMA peak, rank-shard TP MLP fwd+bwd at h=12288,N=8"

# GPT-3 175B layer, one rank of TP = 8
M, H, F = 2048, 12288, 6144
N_PARTIALS = 8
ATT_B, ATT_S, ATT_HL, ATT_D = 1, 2048, 12, 128
V, VN, EMB_TOK = 50304, 8, 8 * 2048


def gemm_flops(m, n, k):
    return 2.0 * m * n * k


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--no-cpu-baseline", action="store_true", help="skip the oracle timing leg")
    p.add_argument("--no-next", action="store_true",
                   help="skip the extra rows timed after the step (PaLM-shaped MLP with recompute, "
                        "cross-entropy, attention backward, sequence parallelism)")
    p.add_argument("--copy-probe", action="store_true",
                   help="after the timed steps, run a plain 256 MiB device-to-device copy three times, "
                        "the calibration kernel for HBM byte counters")
    return p.parse_args()


def cpu_baseline(min_seconds: float = 10.0, max_passes: int = 12):
    """Time the float64 oracle (as it stands) on the GPT-3 MLP shard's forward +
    backward: full passes over the whole batch (M = 2048) of one shard, the same
    work as the GPU's MLP step, repeated until about min_seconds have elapsed."""
    import numpy as np
    from threadpoolctl import threadpool_info

    import oracle
    from oracle.bf16 import bf16_bits_to_f64
    from workloads import CONFIGS, mlp_inputs

    c = CONFIGS["gpt3_mlp_rank_shard"]
    Ms = c["b"] * c["s"]
    inp = mlp_inputs(Ms, c["h"], c["f"], 1, "bf16", c["seed"], c["sigma_x"], c["sigma_w"], c["sigma_dz"],
                     full=False)
    A_i, B_i = inp["shards"][0]
    X, A, B, dZ = (bf16_bits_to_f64(a) for a in (inp["X"], A_i, B_i, inp["dZ"]))
    passes, dt = 0, 0.0
    while passes < max_passes and (passes == 0 or dt < min_seconds):
        t0 = time.perf_counter()
        f = oracle.mlp_fwd_shard(X, A, B)
        oracle.mlp_bwd_shard(X, A, B, f["U"], f["Y"], dZ)
        dt += time.perf_counter() - t0
        passes += 1
    flops = passes * 6 * gemm_flops(Ms, c["f"], c["h"])
    threads = max([d.get("num_threads", 1) for d in threadpool_info() if d.get("user_api") == "blas"] or [1])
    return {"value": round(flops / dt / 1e12, 4), "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "sample": f"float64 oracle MLP fwd+bwd of the GPT-3 rank shard (M=2048, h=12288, f=6144), "
                      f"{passes} full pass(es) in {dt:.2f} s; bf16 storage rounding as on the GPU"}


def traffic_from_profiles(key: str):
    """HBM bytes per launch of one kernel from the committed rocprofv3 counter record
    (profiles/hbm_traffic.json, FETCH_SIZE + WRITE_SIZE scaled by the copy-kernel
    calibration), or None when the record is missing or any kernel source it was
    taken on has changed since."""
    path = os.path.join(ROOT, "profiles", "hbm_traffic.json")
    if not os.path.exists(path):
        return None
    try:
        rec = json.load(open(path))
        for name, digest in rec["source_sha256"].items():
            src = open(os.path.join(ROOT, "attention_shard_math_amd", "csrc", name), "rb").read()
            if hashlib.sha256(src).hexdigest() != digest:
                return None
        return round(rec["kernels"][key]["hbm_bytes_per_launch"])
    except Exception:
        return None


def hbm_ceilings(torch, dev, reps=10):
    """Practical HBM rates of plain runtime kernels at the sizes the bandwidth rows
    move, for reading their fractions against: a fill of the gather's 402.65 MB
    output (write only) and a 1 GiB device copy (read + write, larger than the
    256 MB Infinity Cache). Each figure is `reps` back-to-back launches between
    two HIP events on the current stream, so the cache's write-back is included
    (a lone launch can leave part of its writes in the cache)."""
    out = {}
    fill = torch.empty(16384 * 12288, dtype=torch.bfloat16, device=dev)
    src = torch.empty(1 << 28, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for name, fn, nbytes in (("write_fill_402MB", lambda: fill.zero_(), fill.numel() * 2),
                             ("copy_1GiB", lambda: dst.copy_(src), 2 * src.numel() * 4)):
        fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        out[name] = {"ms": round(ms, 4), "gbs": round(nbytes / ms / 1e6, 1)}
    del fill, src, dst
    return out


def next_rows(tp, torch, dev, randn, reps=5):
    """Rows beyond the step, timed on their own after it: the PaLM 540B MLP shard
    (M = 4096, the page's context; h = 18432, f = 9216), forward with saved U,
    backward with activation recompute (U, Y formed again from X and A_i inside
    mlp_bwd); the PaLM attention shard (6 local heads of 384, s = 4096), forward and
    backward; the
    vocabulary-parallel output layer + cross-entropy of one rank; the attention
    backward (core, and the whole shard); the sequence-parallel LayerNorm,
    all-gather and reduce-scatter of one rank; and, as context, the runtime's
    library GEMM on the six MLP products."""
    Mp, Hp, Fp = 4096, 18432, 9216
    X = randn((Mp, Hp), 1.0, 40)
    A = randn((Hp, Fp), 0.005, 41)
    B = randn((Fp, Hp), 0.005, 42)
    dZ = randn((Mp, Hp), 1.0, 43)
    U = torch.empty(Mp, Fp, dtype=torch.bfloat16, device=dev)
    Y = torch.empty_like(U)
    Z = torch.empty(Mp, Hp, dtype=torch.float32, device=dev)
    dX = torch.empty(Mp, Hp, dtype=torch.float32, device=dev)
    dA = torch.empty(Hp, Fp, dtype=torch.float32, device=dev)
    dB = torch.empty(Fp, Hp, dtype=torch.float32, device=dev)
    ws = torch.empty(tp.mlp_bwd_recompute_workspace(Mp, Hp, Fp), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()
    fwd = lambda: tp.mlp_fwd(X, A, B, Y, Z, U_i=U)
    bwd = lambda: tp.mlp_bwd(X, A, B, None, None, dZ, dX, dA, dB, ws)
    out = {}
    for name, fn, n_gemm in (("palm_mlp_fwd", fwd, 2), ("palm_mlp_bwd_recompute", bwd, 5)):
        for _ in range(2):
            fn()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        tf = n_gemm * gemm_flops(Mp, Fp, Hp) / (ms * 1e-3) / 1e12
        out[name] = {"ms": round(ms, 4), "gemms": n_gemm, "tflops": round(tf, 1),
                     "frac_bf16_peak": round(tf / PEAK_BF16_TFLOPS, 4)}
    del X, A, B, dZ, U, Y, Z, dX, dA, dB, ws
    torch.cuda.empty_cache()

    # PaLM attention shard: 48 heads of 384 over 8 ranks (6 local), s = 4096, h = 18432.
    Sp, Hpa, Hlp, Dp = 4096, 18432, 6, 384
    wp = Hlp * Dp
    Xp = randn((Sp, Hpa), 1.0, 90)
    Wqkvp = randn((Hpa, 3 * wp), 0.005, 91)
    Wop = randn((wp, Hpa), 0.005, 92)
    dOutp = randn((Sp, Hpa), 1.0, 93)
    outpp = torch.empty(Sp, Hpa, dtype=torch.float32, device=dev)
    wsf = torch.empty(tp.attn_fwd_workspace(1, Sp, Hlp, Dp, h=Hpa), dtype=torch.uint8, device=dev)
    QKVp = torch.empty(Sp, 3 * wp, dtype=torch.bfloat16, device=dev)
    Op = torch.empty(Sp, wp, dtype=torch.bfloat16, device=dev)
    lsep = torch.empty(1, Hlp, Sp, dtype=torch.float32, device=dev)
    tp.attn_fwd_train(Xp, Wqkvp, Wop, outpp, QKVp, Op, lsep, 1, Sp, Hlp, Dp, True)
    dXp = torch.empty(Sp, Hpa, dtype=torch.float32, device=dev)
    dWqkvp = torch.empty(Hpa, 3 * wp, dtype=torch.float32, device=dev)
    dWop = torch.empty(wp, Hpa, dtype=torch.float32, device=dev)
    wsbp = torch.empty(tp.attn_bwd_workspace(1, Sp, Hpa, Hlp, Dp), dtype=torch.uint8, device=dev)
    pairs = Sp * (Sp + 1) / 2
    fwd_gf = (2 * 2 * Dp * Hlp * pairs + gemm_flops(Sp, 3 * wp, Hpa) + gemm_flops(Sp, Hpa, wp)) / 1e9
    bwd_gf = (5 * 2 * Dp * Hlp * pairs + 2 * gemm_flops(Sp, wp, Hpa) + 2 * gemm_flops(Sp, 3 * wp, Hpa)) / 1e9
    for name, fn, gf in (
            ("palm_attn_fwd", lambda: tp.attn_fwd(Xp, Wqkvp, Wop, outpp, wsf, 1, Sp, Hlp, Dp, True), fwd_gf),
            ("palm_attn_bwd", lambda: tp.attn_bwd(Xp, Wqkvp, Wop, QKVp, Op, lsep, dOutp, dXp, dWqkvp, dWop, wsbp, 1,
                                                  Sp, Hlp, Dp, True), bwd_gf)):
        for _ in range(2):
            fn()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        tf = gf * 1e9 / (ms * 1e-3) / 1e12
        out[name] = {"ms": round(ms, 4), "gflop": round(gf, 2), "tflops": round(tf, 1),
                     "frac_bf16_peak": round(tf / PEAK_BF16_TFLOPS, 4)}
    del Xp, Wqkvp, Wop, dOutp, outpp, wsf, QKVp, Op, lsep, dXp, dWqkvp, dWop, wsbp
    torch.cuda.empty_cache()

    # Vocabulary-parallel output layer + cross-entropy: one rank's slice of the
    # 50304-entry vocabulary (6288 rows of E), 2048 tokens, h = 12288; then the
    # rank-sum/loss step over 8 slices' partial sums.
    Mv, Hv, Vs, Nv = 2048, 12288, 50304 // 8, 8
    Hh = randn((Mv, Hv), 1.0, 50)
    E = randn((Vs, Hv), 0.02, 51)
    tg = torch.randint(0, 50304, (Mv,), dtype=torch.int32, generator=torch.Generator().manual_seed(52)).to(dev)
    maxs = [torch.empty(Mv, dtype=torch.float32, device=dev) for _ in range(Nv)]
    sums = [torch.empty(Mv, dtype=torch.float32, device=dev) for _ in range(Nv)]
    tls = [torch.empty(Mv, dtype=torch.float32, device=dev) for _ in range(Nv)]
    ws = torch.empty(tp.vocab_ce_workspace(Mv, Hv, 0, Vs), dtype=torch.uint8, device=dev)
    rows = torch.empty(Mv, dtype=torch.float32, device=dev)
    tot = torch.empty(1, dtype=torch.float32, device=dev)
    part = lambda: tp.vocab_ce_partials(Hh, E, tg, 0, Vs, maxs[0], sums[0], tls[0], ws)
    part()
    for i in range(1, Nv):
        maxs[i].copy_(maxs[0])
        sums[i].copy_(sums[0])
        tls[i].zero_()
    loss = lambda: tp.vocab_ce_loss(maxs, sums, tls, rows, tot)
    for name, fn in (("vocab_ce_partials", part), ("vocab_ce_loss", loss)):
        for _ in range(2):
            fn()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        rec = {"ms": round(ms, 4)}
        if name == "vocab_ce_partials":
            tf = gemm_flops(Mv, Vs, Hv) / (ms * 1e-3) / 1e12
            rec.update(tflops=round(tf, 1), frac_bf16_peak=round(tf / PEAK_BF16_TFLOPS, 4))
        out[name] = rec
    del Hh, E, tg, sums, tls, ws, rows, tot
    torch.cuda.empty_cache()

    # Attention at the GPT-3 shard (12 heads x 128, s = 2048, h = 12288): the forward
    # core alone (the step times the whole shard), and the backward, core alone and
    # whole shard (Wo, Wqkv and input-gradient GEMMs).
    Ha, Hla, Da, Sa = 12288, 12, 128, 2048
    wa = Hla * Da
    Xa = randn((Sa, Ha), 1.0, 80)
    Wqkv = randn((Ha, 3 * wa), 0.006, 81)
    Wo = randn((wa, Ha), 0.006, 82)
    dOut = randn((Sa, Ha), 1.0, 83)
    outp = torch.empty(Sa, Ha, dtype=torch.float32, device=dev)
    QKV = torch.empty(Sa, 3 * wa, dtype=torch.bfloat16, device=dev)
    Oa = torch.empty(Sa, wa, dtype=torch.bfloat16, device=dev)
    lse = torch.empty(1, Hla, Sa, dtype=torch.float32, device=dev)
    tp.attn_fwd_train(Xa, Wqkv, Wo, outp, QKV, Oa, lse, 1, Sa, Hla, Da, True)
    dOa = randn((Sa, wa), 1.0, 84)
    dQKV = torch.empty_like(QKV)
    wsc = torch.empty(tp.attn_core_bwd_workspace(1, Sa, Hla, Da), dtype=torch.uint8, device=dev)
    dXa = torch.empty(Sa, Ha, dtype=torch.float32, device=dev)
    dWqkv = torch.empty(Ha, 3 * wa, dtype=torch.float32, device=dev)
    dWo = torch.empty(wa, Ha, dtype=torch.float32, device=dev)
    wsb = torch.empty(tp.attn_bwd_workspace(1, Sa, Ha, Hla, Da), dtype=torch.uint8, device=dev)
    Oc = torch.empty_like(Oa)
    core_fwd_gflop = 2 * 2 * Da * Hla * Sa * (Sa + 1) / 2 / 1e9  # S and P V, causal pairs
    core_gflop = 5 * 2 * Da * Hla * Sa * (Sa + 1) / 2 / 1e9  # dV, dP, dQ, dK + the S recompute, causal pairs
    shard_gflop = core_gflop + (2 * gemm_flops(Sa, wa, Ha) + 2 * gemm_flops(Sa, 3 * wa, Ha)) / 1e9
    for name, fn, gf in (
            ("attn_core_fwd", lambda: tp.attn_core(QKV, Oc, 1, Sa, Hla, Da, True), core_fwd_gflop),
            ("attn_core_bwd", lambda: tp.attn_core_bwd(QKV, Oa, dOa, lse, dQKV, wsc, 1, Sa, Hla, Da, True), core_gflop),
            ("attn_shard_bwd", lambda: tp.attn_bwd(Xa, Wqkv, Wo, QKV, Oa, lse, dOut, dXa, dWqkv, dWo, wsb, 1, Sa,
                                                   Hla, Da, True), shard_gflop)):
        for _ in range(2):
            fn()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        tf = gf * 1e9 / (ms * 1e-3) / 1e12
        out[name] = {"ms": round(ms, 4), "gflop": round(gf, 2), "tflops": round(tf, 1),
                     "frac_bf16_peak": round(tf / PEAK_BF16_TFLOPS, 4)}
    del Xa, Wqkv, Wo, dOut, outp, QKV, Oa, Oc, lse, dOa, dQKV, wsc, dXa, dWqkv, dWo, wsb
    torch.cuda.empty_cache()

    # Sequence parallelism at the GPT-3 shard: one rank's LayerNorm over its 256
    # rows, the all-gather stand-in (8 x 256 rows of bf16), and the reduce-scatter
    # stand-in over 8 fp32 partials [2048, 12288] with dropout and residual.
    Ss, Hs, Ns = 2048, 12288, 8
    rs_rows = Ss // Ns
    Rr = randn((rs_rows, Hs), 1.0, 60, torch.float32)
    gam = randn((Hs,), 0.1, 61, torch.float32) + 1.0
    bet = randn((Hs,), 0.1, 62, torch.float32)
    Ls = [torch.empty(rs_rows, Hs, dtype=torch.bfloat16, device=dev) for _ in range(Ns)]
    Xg = torch.empty(Ss, Hs, dtype=torch.bfloat16, device=dev)
    parts = [randn((Ss, Hs), 1.0, 63 + i, torch.float32) for i in range(Ns)]
    keep = (torch.rand(rs_rows, Hs, generator=torch.Generator().manual_seed(71)) < 0.9).to(torch.uint8).to(dev)
    Ro = torch.empty_like(Rr)
    dYs = randn((rs_rows, Hs), 1.0, 72, torch.float32)
    dRs = randn((rs_rows, Hs), 1.0, 73, torch.float32)
    dXs = torch.empty_like(dYs)
    dgs = torch.empty(Hs, dtype=torch.float32, device=dev)
    dbs = torch.empty_like(dgs)
    lws = torch.empty(tp.layernorm_bwd_workspace(rs_rows, Hs), dtype=torch.uint8, device=dev)
    dZs = torch.empty(rs_rows, Hs, dtype=torch.bfloat16, device=dev)
    sp_rows = (
        ("sp_layernorm", lambda: tp.layernorm(Rr, gam, bet, Ls[0]), rs_rows * Hs * (4 + 2) + 2 * Hs * 4),
        ("sp_layernorm_bwd", lambda: tp.layernorm_bwd(Rr, gam, dYs, dXs, dgs, dbs, lws, dRes=dRs),
         rs_rows * Hs * 16 + 3 * Hs * 4),
        ("sp_dropout_bwd", lambda: tp.sp_dropout_bwd(dYs, dZs, keep=keep, keep_prob=0.9), rs_rows * Hs * 7),
        ("sp_all_gather", lambda: tp.sp_all_gather(Ls, Xg), 2 * Ss * Hs * 2),
        ("sp_reduce_scatter", lambda: tp.sp_reduce_scatter(parts, 3, Rr, Ro, keep=keep, keep_prob=0.9),
         rs_rows * Hs * (4 * Ns + 4 + 1 + 4)),
    )
    for name, fn, nbytes in sp_rows:
        for _ in range(2):
            fn()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        gbs = nbytes / (ms * 1e-3) / 1e9
        out[name] = {"ms": round(ms, 4), "bytes": nbytes, "gbs": round(gbs, 1),
                     "frac_hbm_peak": round(gbs / PEAK_HBM_GBS, 4)}
    del Rr, gam, bet, Ls, Xg, parts, keep, Ro, dYs, dRs, dXs, dgs, dbs, lws, dZs
    torch.cuda.empty_cache()

    # Context, not part of the path: the runtime's library GEMM (hipBLASLt through
    # torch.mm) on the same six MLP products of the GPT-3 shard, on this machine in this
    # run, every operand already contiguous (transposes materialised outside the
    # timing) and bf16 outputs without the epilogues.
    M, H, F = 2048, 12288, 6144
    X = randn((M, H), 1.0, 1)
    A = randn((H, F), 0.006, 2)
    B = randn((F, H), 0.006, 3)
    dZ = randn((M, H), 1.0, 4)
    Y = randn((M, F), 1.0, 5)
    dU = randn((M, F), 1.0, 6)
    Bt, At, Yt, Xt = B.t().contiguous(), A.t().contiguous(), Y.t().contiguous(), X.t().contiguous()
    prods = [(X, A), (Y, B), (dZ, Bt), (Yt, dZ), (Xt, dU), (dU, At)]
    outs = [torch.empty(a.shape[0], b.shape[1], dtype=torch.bfloat16, device=dev) for a, b in prods]

    def six():
        for (a, b), o in zip(prods, outs):
            torch.mm(a, b, out=o)

    for _ in range(2):
        six()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        six()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    tf = 6 * gemm_flops(M, F, H) / (ms * 1e-3) / 1e12
    out["context_library_gemm_mlp6"] = {"ms": round(ms, 4), "tflops": round(tf, 1),
                                        "frac_bf16_peak": round(tf / PEAK_BF16_TFLOPS, 4)}
    del X, A, B, dZ, Y, dU, Bt, At, Yt, Xt, prods, outs
    torch.cuda.empty_cache()
    return out


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library runs one rank's shard on a single MI355X "
              "(no collectives); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch

    import attention_shard_math_amd as tp

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    g = torch.Generator(device=dev)

    def randn(shape, sigma, seed, dtype=torch.bfloat16):
        g.manual_seed(seed)
        return (torch.randn(shape, generator=g, device=dev, dtype=torch.float32) * sigma).to(dtype)

    # ---- MLP shard
    X = randn((M, H), 1.0, 1)
    A = randn((H, F), 0.006, 2)
    B = randn((F, H), 0.006, 3)
    dZ = randn((M, H), 1.0, 4)
    U = torch.empty(M, F, dtype=torch.bfloat16, device=dev)
    Y = torch.empty_like(U)
    Z = torch.empty(M, H, dtype=torch.float32, device=dev)
    dX = torch.empty(M, H, dtype=torch.float32, device=dev)
    dA = torch.empty(H, F, dtype=torch.float32, device=dev)
    dB = torch.empty(F, H, dtype=torch.float32, device=dev)
    ws = torch.empty(tp.mlp_bwd_workspace(M, H, F), dtype=torch.uint8, device=dev)
    # ---- shard-sum partials
    parts = [randn((M * H,), 1.0, 10 + i, torch.float32) for i in range(N_PARTIALS)]
    Zsum = torch.empty(M * H, dtype=torch.float32, device=dev)
    # ---- attention shard
    w = ATT_HL * ATT_D
    Xa = randn((ATT_B * ATT_S, H), 1.0, 20)
    Wqkv = randn((H, 3 * w), 0.006, 21)
    Wo = randn((w, H), 0.006, 22)
    out_att = torch.empty(ATT_B * ATT_S, H, dtype=torch.float32, device=dev)
    ws_att = torch.empty(tp.attn_fwd_workspace(ATT_B, ATT_S, ATT_HL, ATT_D, h=H), dtype=torch.uint8, device=dev)
    # ---- vocab shard 0 of 8
    per = V // VN
    E0 = randn((per, H), 0.02, 30)
    g.manual_seed(31)
    ids = torch.randint(0, V, (EMB_TOK,), generator=g, device=dev, dtype=torch.int32)
    emb = torch.empty(EMB_TOK, H, dtype=torch.bfloat16, device=dev)
    hits = int(((ids >= 0) & (ids < per)).sum().item())

    rows = [
        ("mlp_col_gemm_gelu", lambda: tp.column_linear(X, A, Y, U=U, act="gelu")),
        ("mlp_row_gemm", lambda: tp.row_linear(Y, B, Z)),
        ("mlp_bwd", lambda: tp.mlp_bwd(X, A, B, U, Y, dZ, dX, dA, dB, ws)),
        ("shard_sum", lambda: tp.shard_sum(parts, Zsum)),
        ("attn_shard", lambda: tp.attn_fwd(Xa, Wqkv, Wo, out_att, ws_att, ATT_B, ATT_S, ATT_HL, ATT_D, True)),
        ("vocab_gather", lambda: tp.vocab_embed(ids, E0, 0, per, emb)),
    ]
    flops = {
        "mlp_col_gemm_gelu": gemm_flops(M, F, H),
        "mlp_row_gemm": gemm_flops(M, H, F),
        "mlp_bwd": 4 * gemm_flops(M, F, H),
        "attn_shard": gemm_flops(ATT_B * ATT_S, 3 * w, H) + 2 * 2.0 * ATT_HL * ATT_D * ATT_B * (ATT_S * (ATT_S + 1) / 2)
        + gemm_flops(ATT_B * ATT_S, H, w),
    }
    hbm_bytes = {
        "shard_sum": (N_PARTIALS + 1) * M * H * 4.0,
        "vocab_gather": EMB_TOK * H * 2.0 + hits * H * 2.0 + EMB_TOK * 4.0,
    }

    stream = torch.cuda.current_stream()
    ev = {name: [] for name, _ in rows}

    def step(record):
        for name, fn in rows:
            if record:
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                fn()
                e1.record(stream)
                ev[name].append((e0, e1))
            else:
                fn()

    for _ in range(args.warmup):
        step(False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step(True)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    ms = {name: sum(a.elapsed_time(b) for a, b in ev[name]) / args.steps for name in ev}
    mlp_ms = ms["mlp_col_gemm_gelu"] + ms["mlp_row_gemm"] + ms["mlp_bwd"]
    mlp_flops = flops["mlp_col_gemm_gelu"] + flops["mlp_row_gemm"] + flops["mlp_bwd"]
    value = mlp_flops / (mlp_ms * 1e-3) / 1e12

    breakdown = {}
    for name in ms:
        t = sorted(a.elapsed_time(b) for a, b in ev[name])
        # mean (used for the rates), and the spread of the per-step HIP-event times
        d = {"ms": round(ms[name], 4), "ms_median": round(t[len(t) // 2], 4), "ms_min": round(t[0], 4),
             "ms_p90": round(t[min(len(t) - 1, (9 * len(t)) // 10)], 4)}
        if name in flops:
            tf = flops[name] / (ms[name] * 1e-3) / 1e12
            d.update(tflops=round(tf, 1), frac_bf16_peak=round(tf / PEAK_BF16_TFLOPS, 4))
        if name in hbm_bytes:
            gbs = hbm_bytes[name] / (ms[name] * 1e-3) / 1e9
            d.update(gbs=round(gbs, 1), frac_hbm_peak=round(gbs / PEAK_HBM_GBS, 4))
        breakdown[name] = d

    dom = "mlp_col_gemm_gelu"
    dom_tf = flops[dom] / (ms[dom] * 1e-3) / 1e12
    traffic = traffic_from_profiles(dom)
    rec = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3 / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded normal inputs at the stated shapes and sigmas; uniform token ids)",
        "config": {"workload": "gpt3-175b rank shard, TP=8: MLP fwd+bwd (M=2048, h=12288, f=6144); "
                               "shard-sum 8x[2048,12288] fp32; causal attention 12 heads x 128, s=2048; "
                               "vocab gather 16384 ids into a 6288x12288 shard",
                   "M": M, "h": H, "f": F, "tp": 8, "pct_bf16_peak": round(100 * value / PEAK_BF16_TFLOPS, 2),
                   "mlp_fwd_bwd_gflop": round(mlp_flops / 1e9, 2), "mlp_fwd_bwd_ms": round(mlp_ms, 4)},
        "roofline": {"kernel": "gemm_bf16 column GEMM + erf-GeLU (2048x6144x12288)", "bound": "mfma",
                     "achieved": round(dom_tf, 1), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(dom_tf / PEAK_BF16_TFLOPS, 4), "traffic": traffic},
        "breakdown": breakdown,
    }
    if not args.no_next:
        rec["next_rows"] = next_rows(tp, torch, dev, randn)
        rec["hbm_ceilings"] = hbm_ceilings(torch, dev)
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline()
    if args.copy_probe:
        # Known traffic: 256 MiB read + 256 MiB written per copy (the runtime's blit kernel).
        src = torch.ones(64 << 20, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        rec["copy_probe_bytes_each_way"] = src.numel() * 4
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
