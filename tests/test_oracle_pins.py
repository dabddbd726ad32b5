"""Pins of the CPU oracle to facts that do not come from the oracle itself:
closed forms, textbook constants, brute-force loops on tiny inputs, central
finite differences, the sharding invariants the pages state, library routines
used as cross-checks (tests only) and the pages' worked example."""
import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import bf16 as ob
from oracle import seqpar
from tests import brute
from workloads import CONFIGS, mlp_inputs, shard_cols, shard_rows

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------- bf16 rounding
class TestBf16:
    def test_representable_values_are_fixed_points(self):
        vals = np.array([0.0, 1.0, -2.5, 0.0078125, 3.0 * 2.0 ** -130,  # subnormal
                         2.0 ** -126, (2 - 2.0 ** -7) * 2.0 ** 127, -96.0])
        np.testing.assert_array_equal(ob.round_to_bf16(vals), vals)

    def test_ties_to_even_and_carry(self):
        # 1 + 2^-8 lies half-way between 1 (mantissa 0, even) and 1 + 2^-7 (odd).
        assert ob.round_to_bf16(1.0 + 2.0 ** -8) == 1.0
        # 1 + 3*2^-8 lies half-way between 1 + 2^-7 (odd) and 1 + 2^-6 (even).
        assert ob.round_to_bf16(1.0 + 3 * 2.0 ** -8) == 1.0 + 2.0 ** -6
        # just above a tie rounds up
        assert ob.round_to_bf16(1.0 + 2.0 ** -8 + 2.0 ** -30) == 1.0 + 2.0 ** -7
        # 2 - 2^-8 lies half-way between 2 - 2^-7 (mantissa 127, odd) and 2: carry.
        assert ob.round_to_bf16(2.0 - 2.0 ** -8) == 2.0
        # overflow: the midpoint of the largest finite bf16 and 2^128 goes to inf
        big = (2 - 2.0 ** -7) * 2.0 ** 127
        assert ob.round_to_bf16(big + 2.0 ** 119) == np.inf
        assert ob.round_to_bf16(-(big + 2.0 ** 119)) == -np.inf
        assert ob.round_to_bf16(big + 2.0 ** 118) == big

    def test_bit_patterns(self):
        assert ob.f64_to_bf16_bits(np.array([1.0]))[0] == 0x3F80
        assert ob.f64_to_bf16_bits(np.array([-2.0]))[0] == 0xC000
        assert ob.f64_to_bf16_bits(np.array([2.0 ** -133]))[0] == 0x0001
        assert ob.f64_to_bf16_bits(np.array([np.inf]))[0] == 0x7F80

    def test_all_patterns_roundtrip_and_decode(self):
        bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
        vals = ob.bf16_bits_to_f64(bits)
        # field-by-field decode: sign, 8-bit exponent (bias 127), 7-bit mantissa
        b = bits.astype(np.int64)
        sign = np.where(b >> 15, -1.0, 1.0)
        expo, mant = (b >> 7) & 0xFF, (b & 0x7F).astype(np.float64)
        ref = np.where(expo == 0, sign * np.ldexp(mant / 128.0, -126),
                       sign * np.ldexp(1.0 + mant / 128.0, expo - 127))
        finite = expo != 0xFF
        np.testing.assert_array_equal(vals[finite], ref[finite])
        assert np.all(np.isinf(vals[(expo == 0xFF) & (mant == 0)]))
        assert np.all(np.isnan(vals[(expo == 0xFF) & (mant != 0)]))
        np.testing.assert_array_equal(ob.f64_to_bf16_bits(vals[finite]), bits[finite])

    def test_matches_torch_conversion_on_float32(self):
        rng = np.random.default_rng(7)
        x = np.concatenate([rng.standard_normal(20000).astype(np.float32) * s
                            for s in (1e-3, 1.0, 1e3, 1e-38)])
        ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
        np.testing.assert_array_equal(ob.round_to_bf16(x.astype(np.float64)), ref)


# ---------------------------------------------------------------- GeLU
class TestGelu:
    def test_closed_forms(self):
        assert oracle.gelu(0.0) == 0.0
        # Phi(1) = 0.841344746068542948..., a textbook constant
        assert abs(oracle.gelu(1.0) - 0.8413447460685429) < 1e-15
        assert abs(oracle.gelu_prime(0.0) - 0.5) < 1e-16
        x = np.linspace(-6, 6, 1001)
        # Phi(x) + Phi(-x) = 1  =>  GeLU(x) - GeLU(-x) = x
        np.testing.assert_allclose(oracle.gelu(x) - oracle.gelu(-x), x, rtol=0, atol=1e-14)
        assert abs(oracle.gelu(12.0) - 12.0) < 1e-20
        assert abs(oracle.gelu(-12.0)) < 1e-30

    def test_against_math_erf(self):
        for x in np.linspace(-5, 5, 97):
            assert abs(oracle.gelu(x) - brute.gelu(float(x))) <= 1e-15 * max(1, abs(x))

    def test_derivative_by_central_difference(self):
        x = np.linspace(-5, 5, 201)
        eps = 1e-5
        fd = (oracle.gelu(x + eps) - oracle.gelu(x - eps)) / (2 * eps)
        np.testing.assert_allclose(oracle.gelu_prime(x), fd, rtol=0, atol=1e-9)


# ---------------------------------------------------------------- MLP forward
def _f64(a, dtype):
    return a.astype(np.float64) if dtype == "f32" else ob.bf16_bits_to_f64(a)


class TestMlpForward:
    def test_tiny_mlp_brute_force(self):
        c = CONFIGS["tiny_mlp_fp32"]
        inp = mlp_inputs(c["b"] * c["s"], c["h"], c["f_full"], c["N"], c["dtype"], c["seed"],
                         c["sigma_x"], c["sigma_w"], sigma_dz=None)
        X = _f64(inp["X"], "f32")
        Zsum = np.zeros((X.shape[0], c["h"]))
        for A_i, B_i in inp["shards"]:
            A_i, B_i = _f64(A_i, "f32"), _f64(B_i, "f32")
            z = oracle.mlp_fwd_shard(X, A_i, B_i, matched=False)["Z"]
            zb = np.array(brute.mlp(X.tolist(), A_i.tolist(), B_i.tolist()))
            np.testing.assert_allclose(z, zb, rtol=1e-12, atol=1e-14)
            Zsum += z
        Zfull = np.array(brute.mlp(X.tolist(), _f64(inp["A"], "f32").tolist(),
                                   _f64(inp["B"], "f32").tolist()))
        np.testing.assert_allclose(Zsum, Zfull, rtol=1e-12, atol=1e-14)

    @pytest.mark.parametrize("N", [1, 2, 4, 8])
    def test_sum_of_partials_is_unsharded_mlp(self, N):
        inp = mlp_inputs(24, 64, 256, N, "f32", 11, 1.0, 0.05, sigma_dz=None)
        X, A, B = (inp[k].astype(np.float64) for k in "XAB")
        Z = sum(oracle.mlp_fwd_shard(X, a.astype(np.float64), b.astype(np.float64),
                                     matched=False)["Z"] for a, b in inp["shards"])
        ref = oracle.mlp_fwd_full(X, A, B)
        assert np.max(np.abs(Z - ref)) <= 1e-12 * np.max(np.abs(ref))
        if N == 1:
            np.testing.assert_array_equal(
                oracle.mlp_fwd_shard(X, A, B, matched=False)["Z"], ref)

    def test_matched_partials_sum_to_matched_unsharded(self):
        # bf16 rounding of GeLU(XA) is elementwise, so splitting the columns
        # before or after rounding gives the same rounded activations.
        inp = mlp_inputs(24, 64, 256, 4, "bf16", 15, 1.0, 0.05, sigma_dz=None)
        X, A, B = (ob.bf16_bits_to_f64(inp[k]) for k in "XAB")
        Z = sum(oracle.mlp_fwd_shard(X, ob.bf16_bits_to_f64(a), ob.bf16_bits_to_f64(b))["Z"]
                for a, b in inp["shards"])
        ref = oracle.mlp_fwd_full(X, A, B, matched=True)
        assert np.max(np.abs(Z - ref)) <= 1e-12 * np.max(np.abs(ref))
        assert np.max(np.abs(ref - oracle.mlp_fwd_full(X, A, B))) > 0  # the rounding is visible

    def test_column_shards_concatenate(self):
        inp = mlp_inputs(16, 32, 128, 4, "f32", 12, 1.0, 0.1, sigma_dz=None)
        X, A = inp["X"].astype(np.float64), inp["A"].astype(np.float64)
        U = np.concatenate([oracle.mlp_fwd_shard(X, a.astype(np.float64),
                                                 b.astype(np.float64), matched=False)["U"]
                            for a, b in inp["shards"]], axis=1)
        Ub = np.array(brute.matmul(X.tolist(), A.tolist()))
        np.testing.assert_allclose(U, Ub, rtol=1e-13, atol=1e-13)

    def test_linear_in_B(self):
        rng = np.random.default_rng(3)
        X, A = rng.standard_normal((8, 16)), rng.standard_normal((16, 32))
        B1, B2 = rng.standard_normal((32, 16)), rng.standard_normal((32, 16))
        z = lambda B: oracle.mlp_fwd_shard(X, A, B, matched=False)["Z"]
        np.testing.assert_allclose(z(B1 + B2), z(B1) + z(B2), rtol=1e-12, atol=1e-12)

    def test_matched_mode_rounds_only_storage_points(self):
        inp = mlp_inputs(8, 64, 128, 1, "bf16", 13, 1.0, 0.05, sigma_dz=None, full=False)
        X, A, B = (ob.bf16_bits_to_f64(inp[k]) for k in "XAB")
        m = oracle.mlp_fwd_shard(X, A, B, matched=True)
        np.testing.assert_array_equal(m["U"], ob.round_to_bf16(X @ A))
        np.testing.assert_array_equal(m["Y"], ob.round_to_bf16(oracle.gelu(X @ A)))
        np.testing.assert_allclose(m["Z"], m["Y"] @ B, rtol=1e-14)

    def test_sampled_rows_equal_full(self):
        inp = mlp_inputs(40, 64, 96, 1, "bf16", 14, 1.0, 0.05, sigma_dz=None, full=False)
        X, A, B = (ob.bf16_bits_to_f64(inp[k]) for k in "XAB")
        full = oracle.mlp_fwd_shard(X, A, B)
        rows = np.array([0, 7, 39])
        part = oracle.mlp_fwd_rows(X, A, B, rows)
        for k in ("U", "Y", "Z"):
            np.testing.assert_allclose(part[k], full[k][rows], rtol=1e-14, atol=1e-15)


# ---------------------------------------------------------------- MLP backward
class TestMlpBackward:
    def _tiny(self, N=2, seed=21):
        inp = mlp_inputs(6, 8, 32, N, "f32", seed, 1.0, 0.3, sigma_dz=1.0)
        return {k: (v.astype(np.float64) if isinstance(v, np.ndarray) else v)
                for k, v in inp.items()}

    def test_finite_differences(self):
        inp = self._tiny()
        X, dZ = inp["X"], inp["dZ"]
        eps = 1e-6
        for A_i, B_i in inp["shards"]:
            A_i, B_i = A_i.astype(np.float64), B_i.astype(np.float64)
            f = oracle.mlp_fwd_shard(X, A_i, B_i, matched=False)
            g = oracle.mlp_bwd_shard(X, A_i, B_i, f["U"], f["Y"], dZ, matched=False)

            def L(Xp=X, Ap=A_i, Bp=B_i):  # the rank's share of <dZ, Z>
                return float(np.sum(dZ * oracle.mlp_fwd_shard(Xp, Ap, Bp, matched=False)["Z"]))

            for (arr, key, idx) in [(X, "dX", (1, 3)), (X, "dX", (5, 0)),
                                    (A_i, "dA", (2, 7)), (A_i, "dA", (7, 0)),
                                    (B_i, "dB", (3, 5)), (B_i, "dB", (15, 7))]:
                p, m = arr.copy(), arr.copy()
                p[idx] += eps
                m[idx] -= eps
                kw = {"dX": "Xp", "dA": "Ap", "dB": "Bp"}[key]
                fd = (L(**{kw: p}) - L(**{kw: m})) / (2 * eps)
                assert abs(fd - g[key][idx]) <= 1e-7 * max(1.0, abs(fd)), (key, idx, fd, g[key][idx])

    @pytest.mark.parametrize("N", [1, 2, 4])
    def test_shard_gradients_assemble_the_unsharded_ones(self, N):
        inp = self._tiny(N=N, seed=22)
        X, A, B, dZ = inp["X"], inp["A"], inp["B"], inp["dZ"]
        full = oracle.mlp_bwd_full(X, A, B, dZ)
        parts = []
        for A_i, B_i in inp["shards"]:
            A_i, B_i = A_i.astype(np.float64), B_i.astype(np.float64)
            f = oracle.mlp_fwd_shard(X, A_i, B_i, matched=False)
            parts.append(oracle.mlp_bwd_shard(X, A_i, B_i, f["U"], f["Y"], dZ, matched=False))
        np.testing.assert_allclose(sum(p["dX"] for p in parts), full["dX"], rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(np.concatenate([p["dA"] for p in parts], 1), full["dA"],
                                   rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(np.concatenate([p["dB"] for p in parts], 0), full["dB"],
                                   rtol=1e-12, atol=1e-13)

    def test_against_torch_autograd(self):
        inp = self._tiny(N=1, seed=23)
        X, A, B, dZ = (torch.tensor(inp[k], dtype=torch.float64, requires_grad=True)
                       for k in ("X", "A", "B", "dZ"))
        Z = torch.nn.functional.gelu(X @ A) @ B  # exact (erf) GeLU by default
        Z.backward(dZ.detach())
        full = oracle.mlp_bwd_full(inp["X"], inp["A"], inp["B"], inp["dZ"])
        for key, t in (("dX", X), ("dA", A), ("dB", B)):
            np.testing.assert_allclose(full[key], t.grad.numpy(), rtol=1e-12, atol=1e-13)

    def test_sampled_backward_equals_full(self):
        inp = mlp_inputs(24, 32, 48, 1, "bf16", 24, 1.0, 0.1, sigma_dz=1.0, full=False)
        X, A, B, dZ = (ob.bf16_bits_to_f64(inp[k]) for k in ("X", "A", "B", "dZ"))
        f = oracle.mlp_fwd_shard(X, A, B)
        g = oracle.mlp_bwd_shard(X, A, B, f["U"], f["Y"], dZ)
        rows, cols = np.array([0, 5, 23]), np.array([1, 30, 47])
        s = oracle.mlp_bwd_cols(X, A, B, dZ, rows, cols)
        np.testing.assert_allclose(s["dU_cols"], g["dU"][:, cols], rtol=1e-13, atol=1e-14)
        np.testing.assert_allclose(s["dA_cols"], g["dA"][:, cols], rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(s["dB_rows"], g["dB"][cols, :], rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(s["dX_rows"], g["dX"][rows, :], rtol=1e-12, atol=1e-13)


# ---------------------------------------------------------------- shard sum
class TestShardSum:
    def test_integer_valued_partials_sum_exactly(self):
        rng = np.random.default_rng(31)
        parts = [rng.integers(-1000, 1000, 777).astype(np.float32) for _ in range(8)]
        exact = np.sum(np.stack(parts).astype(np.int64), axis=0)
        np.testing.assert_array_equal(oracle.shard_sum_f32_ordered(parts), exact)
        np.testing.assert_array_equal(oracle.shard_sum_f64(parts), exact)

    def test_single_partial_is_a_copy(self):
        p = np.random.default_rng(32).standard_normal(100).astype(np.float32)
        np.testing.assert_array_equal(oracle.shard_sum_f32_ordered([p]), p)

    def test_order_is_left_to_right_in_float32(self):
        # (1e8 + 1) rounds back to 1e8 in float32, so the ordered sum loses the 1.
        parts = [np.array([1e8], np.float32), np.array([1.0], np.float32),
                 np.array([-1e8], np.float32)]
        assert oracle.shard_sum_f32_ordered(parts)[0] == 0.0
        assert oracle.shard_sum_f64(parts)[0] == 1.0
        rev = oracle.shard_sum_f32_ordered(parts[::-1])
        assert rev[0] == 0.0 and oracle.shard_sum_f32_ordered([parts[0], parts[2], parts[1]])[0] == 1.0

    def test_bf16_disjoint_supports_are_exact(self):
        rng = np.random.default_rng(33)
        full = ob.f64_to_bf16_bits(rng.standard_normal(64))
        owner = rng.integers(0, 4, 64)
        parts = [np.where(owner == i, full, np.uint16(0)).astype(np.uint16) for i in range(4)]
        np.testing.assert_array_equal(oracle.shard_sum_bf16_ordered(parts), full)


# ---------------------------------------------------------------- attention
def _rand(rng, *shape, scale=1.0):
    return rng.standard_normal(shape) * scale


class TestAttention:
    def test_brute_force(self):
        rng = np.random.default_rng(41)
        b, s, H, d, h = 2, 5, 2, 4, 8
        X, Wqkv, Wo = _rand(rng, b * s, h), _rand(rng, h, 3 * H * d, scale=0.5), _rand(rng, H * d, h)
        for causal in (True, False):
            r = oracle.attn_shard(X, Wqkv, Wo, b, s, H, d, causal, matched=False)
            QKV = brute.matmul(X.tolist(), Wqkv.tolist())
            O = [[0.0] * (H * d) for _ in range(b * s)]
            for bi in range(b):
                for j in range(H):
                    q = [row[j * d:(j + 1) * d] for row in QKV[bi * s:(bi + 1) * s]]
                    k = [row[H * d + j * d:H * d + (j + 1) * d] for row in QKV[bi * s:(bi + 1) * s]]
                    v = [row[2 * H * d + j * d:2 * H * d + (j + 1) * d] for row in QKV[bi * s:(bi + 1) * s]]
                    o = brute.attention_head(q, k, v, causal)
                    for t in range(s):
                        O[bi * s + t][j * d:(j + 1) * d] = o[t]
            out = brute.matmul(O, Wo.tolist())
            np.testing.assert_allclose(r["out"], np.array(out), rtol=1e-12, atol=1e-12)

    def test_first_row_sees_only_itself(self):
        rng = np.random.default_rng(42)
        b, s, H, d, h = 1, 7, 3, 4, 12
        X, Wqkv, Wo = _rand(rng, s, h), _rand(rng, h, 3 * H * d), _rand(rng, H * d, h)
        r = oracle.attn_shard(X, Wqkv, Wo, b, s, H, d, True, matched=False)
        np.testing.assert_allclose(r["O"][0], r["V"][0], rtol=1e-14, atol=1e-14)

    def test_zero_queries_give_prefix_means(self):
        rng = np.random.default_rng(43)
        b, s, H, d, h = 2, 6, 2, 4, 8
        X, Wqkv, Wo = _rand(rng, b * s, h), _rand(rng, h, 3 * H * d), _rand(rng, H * d, h)
        Wqkv[:, :H * d] = 0.0
        r = oracle.attn_shard(X, Wqkv, Wo, b, s, H, d, True, matched=False)
        V = r["V"]
        for bi in range(b):
            Vs = V[bi * s:(bi + 1) * s]
            pref = np.cumsum(Vs, axis=0) / np.arange(1, s + 1)[:, None]
            np.testing.assert_allclose(r["O"][bi * s:(bi + 1) * s], pref, rtol=1e-13, atol=1e-13)

    @pytest.mark.parametrize("N", [2, 4, 8])
    def test_head_shards_sum_to_full_mha(self, N):
        rng = np.random.default_rng(44 + N)
        b, s, H, d = 2, 9, 8, 8
        h = H * d
        X = _rand(rng, b * s, h)
        Wq, Wk, Wv = (_rand(rng, h, h, scale=h ** -0.5) for _ in range(3))
        Wo = _rand(rng, h, h, scale=h ** -0.5)
        full = oracle.mha_full(X, Wq, Wk, Wv, Wo, b, s, H, d)
        Hl = H // N
        tot = np.zeros_like(full)
        for i in range(N):
            cols = slice(i * Hl * d, (i + 1) * Hl * d)
            Wqkv_i = np.concatenate([Wq[:, cols], Wk[:, cols], Wv[:, cols]], axis=1)
            tot += oracle.attn_shard(X, Wqkv_i, Wo[cols, :], b, s, Hl, d, matched=False)["out"]
        np.testing.assert_allclose(tot, full, rtol=1e-12, atol=1e-12)

    def test_head_permutation_invariance(self):
        rng = np.random.default_rng(45)
        b, s, H, d, h = 1, 8, 4, 4, 16
        X, Wqkv, Wo = _rand(rng, s, h), _rand(rng, h, 3 * H * d, scale=0.3), _rand(rng, H * d, h)
        perm = [2, 0, 3, 1]
        cols = np.concatenate([np.arange(j * d, (j + 1) * d) for j in perm])
        Wqkv_p = np.concatenate([Wqkv[:, blk * H * d + cols] for blk in range(3)], axis=1)
        a = oracle.attn_shard(X, Wqkv, Wo, b, s, H, d, matched=False)["out"]
        p = oracle.attn_shard(X, Wqkv_p, Wo[cols, :], b, s, H, d, matched=False)["out"]
        np.testing.assert_allclose(a, p, rtol=1e-12, atol=1e-12)

    def test_against_torch_sdpa(self):
        rng = np.random.default_rng(46)
        b, s, H, d = 2, 16, 3, 8
        Q, K, V = (_rand(rng, b * s, H * d) for _ in range(3))
        O = oracle.attn_core(Q, K, V, b, s, H, d, causal=True)
        t = lambda A: torch.tensor(A).reshape(b, s, H, d).transpose(1, 2)
        ref = torch.nn.functional.scaled_dot_product_attention(t(Q), t(K), t(V), is_causal=True)
        np.testing.assert_allclose(O, ref.transpose(1, 2).reshape(b * s, H * d).numpy(),
                                   rtol=1e-12, atol=1e-12)

    def test_sampled_rows_equal_full(self):
        rng = np.random.default_rng(47)
        b, s, H, d, h = 2, 12, 2, 8, 16
        X = ob.round_to_bf16(_rand(rng, b * s, h))
        Wqkv, Wo = ob.round_to_bf16(_rand(rng, h, 3 * H * d, scale=0.2)), ob.round_to_bf16(_rand(rng, H * d, h))
        full = oracle.attn_shard(X, Wqkv, Wo, b, s, H, d)
        rows = np.array([0, 5, 12, 23])
        part = oracle.attn_shard_rows(X, Wqkv, Wo, b, s, H, d, rows)
        np.testing.assert_allclose(part["out"], full["out"][rows], rtol=1e-12, atol=1e-13)


# ---------------------------------------------------------------- embedding
def _read_golden_split():
    ids, vocab, ranks = None, None, []
    with open(os.path.join(GOLDEN, "vocab_split_example.txt")) as fh:
        for line in fh:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            key, *rest = line.split()
            if key == "ids":
                ids = [int(x) for x in rest]
            elif key == "vocab":
                vocab = int(rest[0])
            elif key == "rank":
                lo, hi, colon, *rows = rest
                assert colon == ":"
                ranks.append((int(lo), int(hi), [int(r) for r in rows]))
    return ids, vocab, ranks


class TestEmbedding:
    def test_pages_worked_example(self):
        ids, vocab, ranks = _read_golden_split()
        h = 3
        E = np.arange(vocab * h, dtype=np.int64).reshape(vocab, h) + 1  # no zero rows
        total = np.zeros((len(ids), h), np.int64)
        for lo, hi, rows in ranks:
            out = oracle.vocab_embed_shard(ids, E[lo:hi], lo, hi)
            for t, r in enumerate(rows):
                want = np.zeros(h, np.int64) if r < 0 else E[lo:hi][r]
                np.testing.assert_array_equal(out[t], want)
            total += out
        np.testing.assert_array_equal(total, E[ids])

    def test_shards_assemble_lookup_and_misses_are_zero(self):
        rng = np.random.default_rng(51)
        v, h, N = 96, 5, 8
        E = ob.f64_to_bf16_bits(rng.standard_normal((v, h)) * 0.02)
        assert not np.any(E == 0x8000)  # no -0.0 entries (so adding +0.0 rows is exact)
        ids = rng.integers(-10, v + 10, 200).astype(np.int32)
        outs = [oracle.vocab_embed_shard(ids, E[i * v // N:(i + 1) * v // N], i * v // N, (i + 1) * v // N)
                for i in range(N)]
        got = np.zeros((ids.size, h), np.uint16)
        for o in outs:
            nz = o != 0
            assert not np.any(nz & (got != 0))  # at most one rank contributes a row
            got = np.where(nz, o, got)
        inr = (ids >= 0) & (ids < v)
        np.testing.assert_array_equal(got[inr], E[ids[inr]])
        assert not np.any(got[~inr])


# ---------------------------------------------------------------- vocab-parallel cross-entropy
class TestVocabCrossEntropy:
    @staticmethod
    def _case(seed, M=6, h=5, v=24):
        rng = np.random.default_rng(seed)
        H = rng.standard_normal((M, h))
        E = rng.standard_normal((v, h)) * 0.5
        t = rng.integers(0, v, M)
        return H, E, t

    def test_zero_table_gives_log_v_per_row(self):
        # closed form: every logit is 0, so sum(e) = v and each row's loss is log v
        M, h, v = 7, 4, 30
        H = np.random.default_rng(60).standard_normal((M, h))
        r = oracle.vocab_ce_sharded(H, np.zeros((v, h)), np.arange(M) % v, 3)
        np.testing.assert_allclose(r["loss_rows"], np.log(v), rtol=0, atol=1e-14)
        assert abs(r["loss"] - M * np.log(v)) < 1e-12

    def test_brute_force_loops(self):
        H, E, t = self._case(61, M=4, h=3, v=9)
        N = 3
        r = oracle.vocab_ce_sharded(H, E, t, N)
        for m in range(H.shape[0]):
            S = 0.0
            for n in range(E.shape[0]):
                dot = 0.0
                for k in range(H.shape[1]):
                    dot += H[m, k] * E[n, k]
                S += math.exp(dot)
            lt = sum(H[m, k] * E[t[m], k] for k in range(H.shape[1]))
            assert abs(r["loss_rows"][m] - (math.log(S) - lt)) < 1e-12

    @pytest.mark.parametrize("N", [1, 2, 4, 8])
    def test_sharded_equals_full_log_softmax(self, N):
        # library cross-check: full-vocabulary cross-entropy through scipy's
        # max-shifted logsumexp (a different summation route)
        from scipy.special import logsumexp
        H, E, t = self._case(62 + N, M=10, h=6, v=40)
        logits = H @ E.T
        want = logsumexp(logits, axis=1) - logits[np.arange(10), t]
        r = oracle.vocab_ce_sharded(H, E, t, N)
        np.testing.assert_allclose(r["loss_rows"], want, rtol=1e-12, atol=1e-12)
        assert abs(r["loss"] - want.sum()) < 1e-10

    @pytest.mark.parametrize("N", [1, 3, 5])
    def test_combine_of_column_slices_is_the_full_cross_entropy(self, N):
        # per-slice sums of exp and target logits, formed here from a logits matrix cut
        # into N column slices, combine to scipy's cross-entropy over all the columns
        from scipy.special import log_softmax
        rng = np.random.default_rng(80 + N)
        logits = rng.standard_normal((7, 30)) * 3
        t = rng.integers(0, 30, 7)
        cuts = np.linspace(0, 30, N + 1).astype(int)
        sums, tls = [], []
        for lo, hi in zip(cuts[:-1], cuts[1:]):
            sums.append(np.exp(logits[:, lo:hi]).sum(axis=1))
            tls.append(np.where((t >= lo) & (t < hi), logits[np.arange(7), np.clip(t, lo, hi - 1)], 0.0))
        r = oracle.vocab_ce_combine(sums, tls)
        want = -log_softmax(logits, axis=1)[np.arange(7), t]
        np.testing.assert_allclose(r["loss_rows"], want, rtol=1e-12, atol=1e-12)
        assert abs(r["loss"] - want.sum()) < 1e-10

    def test_shift_invariance(self):
        # adding one vector u to every row of E adds H u to every logit of a row,
        # which the softmax cancels
        H, E, t = self._case(70, M=8, h=5, v=32)
        u = np.random.default_rng(71).standard_normal(5)
        a = oracle.vocab_ce_sharded(H, E, t, 4)
        b = oracle.vocab_ce_sharded(H, E + u, t, 4)
        np.testing.assert_allclose(a["loss_rows"], b["loss_rows"], rtol=1e-10, atol=1e-10)

    def test_exactly_one_rank_holds_each_target(self):
        H, E, t = self._case(72, M=12, h=4, v=48)
        N, v = 4, 48
        parts = [oracle.vocab_ce_partials(H, E[i * v // N:(i + 1) * v // N], t, i * v // N, (i + 1) * v // N)
                 for i in range(N)]
        logits = H @ E.T
        for m in range(12):
            holders = [i for i in range(N) if i * v // N <= t[m] < (i + 1) * v // N]
            assert len(holders) == 1
            for i, p in enumerate(parts):
                if i in holders:
                    assert abs(p["tlogit"][m] - logits[m, t[m]]) < 1e-12
                else:
                    assert p["tlogit"][m] == 0.0


class TestSequenceParallel:
    """Sequence-parallel MLP block [www.discosf.com/news/5875844, 2.3] with the
    all-reduce split into reduce-scatter + all-gather [m.youleyou.com/wenzhang/
    3143730, 二、§2.2]."""

    def _ln_inputs(self, s, h, seed):
        rng = np.random.default_rng(seed)
        R = rng.standard_normal((s, h)) * 3.0 + 0.5
        gamma = 1.0 + 0.1 * rng.standard_normal(h)
        beta = 0.1 * rng.standard_normal(h)
        return R, gamma, beta

    def test_layernorm_brute_force(self):
        R, g, b = self._ln_inputs(5, 7, 11)
        got = seqpar.layernorm(R, g, b, 1e-5)
        want = np.array(brute.layernorm(R.tolist(), g.tolist(), b.tolist(), 1e-5))
        np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-12)

    def test_layernorm_torch(self):
        R, g, b = self._ln_inputs(16, 96, 12)
        want = torch.nn.functional.layer_norm(torch.from_numpy(R), (96,), torch.from_numpy(g),
                                              torch.from_numpy(b), eps=1e-5).numpy()
        np.testing.assert_allclose(seqpar.layernorm(R, g, b), want, rtol=1e-12, atol=1e-12)

    def test_layernorm_moments_and_affine_invariance(self):
        R, _, _ = self._ln_inputs(8, 64, 13)
        ones, zeros = np.ones(64), np.zeros(64)
        y = seqpar.layernorm(R, ones, zeros, eps=0.0)
        np.testing.assert_allclose(y.mean(axis=1), 0.0, atol=1e-13)
        np.testing.assert_allclose((y ** 2).mean(axis=1), 1.0, rtol=1e-12)
        # LN(a x + c) with eps a^2 equals LN(x) with eps
        a, c = 7.5, -3.25
        np.testing.assert_allclose(seqpar.layernorm(a * R + c, ones, zeros, eps=1e-5 * a * a),
                                   seqpar.layernorm(R, ones, zeros, eps=1e-5), rtol=1e-11, atol=1e-12)

    def test_gather_and_scatter_are_the_halves_of_an_all_reduce(self):
        rng = np.random.default_rng(14)
        N, s, h = 4, 12, 5
        parts = [rng.standard_normal((s, h)) for _ in range(N)]
        full = oracle.shard_sum_f64(parts)
        scattered = [seqpar.reduce_scatter(parts, N, i) for i in range(N)]
        np.testing.assert_array_equal(seqpar.all_gather(scattered), full)
        for i in range(N):
            np.testing.assert_array_equal(scattered[i], full[3 * i:3 * (i + 1)])

    @pytest.mark.parametrize("s,N", [(16, 1), (16, 2), (16, 4), (24, 8)])
    def test_row_slices_partition_the_rows_in_rank_order(self, s, N):
        rows = [np.arange(s)[seqpar.row_slice(s, N, i)] for i in range(N)]
        assert all(len(r) == s // N for r in rows)
        np.testing.assert_array_equal(np.concatenate(rows), np.arange(s))

    def test_dropout_residual(self):
        rng = np.random.default_rng(15)
        R, O = rng.standard_normal((4, 6)), rng.standard_normal((4, 6))
        np.testing.assert_array_equal(seqpar.dropout_residual(R, O), R + O)
        np.testing.assert_array_equal(seqpar.dropout_residual(R, O, np.zeros((4, 6), np.uint8), 0.9), R)
        np.testing.assert_allclose(seqpar.dropout_residual(R, O, np.ones((4, 6), np.uint8), 0.5), R + 2 * O)
        keep = (rng.random((4, 6)) < 0.5).astype(np.uint8)
        want = [[R[r][c] + (O[r][c] / 0.8 if keep[r][c] else 0.0) for c in range(6)] for r in range(4)]
        np.testing.assert_allclose(seqpar.dropout_residual(R, O, keep, 0.8), want, rtol=1e-15)

    @pytest.mark.parametrize("N", [1, 2, 4])
    def test_sequence_parallel_equals_tensor_parallel(self, N):
        s, h, f_full = 16, 32, 128
        R, g, b = self._ln_inputs(s, h, 16 + N)
        inp = mlp_inputs(s, h, f_full, N, "f32", 17, 1.0, 0.05, None)
        shards = [(A.astype(np.float64), B.astype(np.float64)) for A, B in inp["shards"]]
        keep = (np.random.default_rng(18).random((s, h)) < 0.9).astype(np.uint8)
        for matched in (False, True):
            sp = seqpar.sp_mlp_block(R, g, b, shards, keep, 0.9, matched=matched)
            tp_ = seqpar.tp_mlp_block(R, g, b, shards, keep, 0.9, matched=matched)
            np.testing.assert_array_equal(sp["X"], tp_["X"])
            np.testing.assert_allclose(sp["R_out"], tp_["R_out"], rtol=1e-13, atol=1e-13)
        # unsharded: LayerNorm, GeLU(XA)B, dropout, residual written out directly
        X = seqpar.layernorm(R, g, b)
        Z = np.array(brute.mlp(X.tolist(), inp["A"].astype(np.float64).tolist(), inp["B"].astype(np.float64).tolist()))
        want = R + np.where(keep != 0, Z / 0.9, 0.0)
        np.testing.assert_allclose(seqpar.sp_mlp_block(R, g, b, shards, keep, 0.9, matched=False)["R_out"], want,
                                   rtol=1e-11, atol=1e-11)


class TestAttentionBackward:
    """Attention backward [m.youleyou.com/wenzhang/3143730, 三、§3.2]: the chain rule
    through per-head causal softmax attention, pinned against torch's float64
    autograd, central finite differences, and the head-sharding identities."""

    def _qkv(self, seed, b, s, H, d, scale=0.7):
        rng = np.random.default_rng(seed)
        return [rng.standard_normal((b * s, H * d)) * scale for _ in range(4)]

    @pytest.mark.parametrize("causal", [True, False])
    def test_torch_autograd(self, causal):
        b, s, H, d = 2, 9, 3, 8
        Q, K, V, dO = self._qkv(61, b, s, H, d)
        dQ, dK, dV = oracle.attn_core_bwd(Q, K, V, dO, b, s, H, d, causal)
        tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (Q, K, V))
        outs = []
        for bi in range(b):
            r = slice(bi * s, (bi + 1) * s)
            for j in range(H):
                c = slice(j * d, (j + 1) * d)
                outs.append((torch.nn.functional.scaled_dot_product_attention(
                    tq[r, c][None], tk[r, c][None], tv[r, c][None], is_causal=causal)[0] *
                    torch.from_numpy(dO[r, c])).sum())
        torch.stack(outs).sum().backward()
        for g, t in ((dQ, tq), (dK, tk), (dV, tv)):
            np.testing.assert_allclose(g, t.grad.numpy(), rtol=1e-10, atol=1e-12)

    def test_finite_differences(self):
        b, s, H, d = 1, 5, 1, 4
        Q, K, V, dO = self._qkv(62, b, s, H, d)
        grads = oracle.attn_core_bwd(Q, K, V, dO, b, s, H, d, True)
        eps = 1e-6
        for which in range(3):
            for (i, j) in [(0, 0), (2, 3), (4, 1)]:
                args = [Q.copy(), K.copy(), V.copy()]
                args[which][i, j] += eps
                fp = (oracle.attn_core(*args, b, s, H, d, True) * dO).sum()
                args[which][i, j] -= 2 * eps
                fm = (oracle.attn_core(*args, b, s, H, d, True) * dO).sum()
                assert abs((fp - fm) / (2 * eps) - grads[which][i, j]) < 1e-7

    def test_last_key_and_first_query(self):
        """Causal: the last key is seen only by the last query, so dV of the last
        key is P[s-1, s-1] dO[s-1]; the first query attends only to the first key,
        so its dQ is zero (softmax of one entry is constant)."""
        b, s, H, d = 1, 6, 1, 4
        Q, K, V, dO = self._qkv(63, b, s, H, d)
        dQ, dK, dV = oracle.attn_core_bwd(Q, K, V, dO, b, s, H, d, True)
        lse = oracle.attn_lse(Q, K, b, s, H, d, True)[0, 0]
        p_last = np.exp(Q[-1] @ K[-1] / np.sqrt(d) - lse[-1])
        np.testing.assert_allclose(dV[-1], p_last * dO[-1], rtol=1e-12)
        np.testing.assert_allclose(dQ[0], 0.0, atol=1e-15)
        # lse of the first query is its own scaled score
        np.testing.assert_allclose(lse[0], Q[0] @ K[0] / np.sqrt(d), rtol=1e-12)

    @pytest.mark.parametrize("causal", [True, False])
    def test_row_term_from_the_output(self, causal):
        """rowsum(P * dP) = rowsum(dO * O) for O = P V: given the exact O, the
        stored-output form of the backward reproduces the definition; given a
        perturbed O, dV is unchanged and dQ, dK move."""
        b, s, H, d = 2, 7, 2, 8
        Q, K, V, dO = self._qkv(65, b, s, H, d)
        O = oracle.attn_core(Q, K, V, b, s, H, d, causal)
        ref = oracle.attn_core_bwd(Q, K, V, dO, b, s, H, d, causal)
        via_o = oracle.attn_core_bwd(Q, K, V, dO, b, s, H, d, causal, O=O)
        for g, r in zip(via_o, ref):
            np.testing.assert_allclose(g, r, rtol=1e-11, atol=1e-13)
        moved = oracle.attn_core_bwd(Q, K, V, dO, b, s, H, d, causal, O=O + 1e-3)
        np.testing.assert_array_equal(moved[2], ref[2])
        assert np.abs(moved[0] - ref[0]).max() > 1e-6 and np.abs(moved[1] - ref[1]).max() > 1e-6

    def test_shards_sum_to_full_mha_backward(self):
        rng = np.random.default_rng(64)
        b, s, Hh, d, N = 1, 6, 4, 4, 2
        h = Hh * d
        X = rng.standard_normal((b * s, h))
        Wq, Wk, Wv = (rng.standard_normal((h, h)) * 0.3 for _ in range(3))
        Wo = rng.standard_normal((h, h)) * 0.3
        dOut = rng.standard_normal((b * s, h))
        tX = torch.tensor(X, requires_grad=True)
        tW = [torch.tensor(w, requires_grad=True) for w in (Wq, Wk, Wv, Wo)]
        Qf, Kf, Vf = (tX @ w for w in tW[:3])
        heads = []
        for j in range(Hh):
            c = slice(j * d, (j + 1) * d)
            heads.append(torch.nn.functional.scaled_dot_product_attention(Qf[:, c][None], Kf[:, c][None],
                                                                          Vf[:, c][None], is_causal=True)[0])
        ((torch.cat(heads, 1) @ tW[3]) * torch.from_numpy(dOut)).sum().backward()
        Hl = Hh // N
        dX = np.zeros_like(X)
        for i in range(N):
            cols = slice(i * Hl * d, (i + 1) * Hl * d)
            Wqkv_i = np.concatenate([Wq[:, cols], Wk[:, cols], Wv[:, cols]], axis=1)
            r = oracle.attn_shard_bwd(X, Wqkv_i, Wo[cols], dOut, b, s, Hl, d, True, matched=False)
            dX += r["dX"]
            np.testing.assert_allclose(r["dWo"], tW[3].grad.numpy()[cols], rtol=1e-10, atol=1e-12)
            w = Hl * d
            for k, tw in enumerate(tW[:3]):
                np.testing.assert_allclose(r["dWqkv"][:, k * w:(k + 1) * w], tw.grad.numpy()[:, cols],
                                           rtol=1e-10, atol=1e-12)
        np.testing.assert_allclose(dX, tX.grad.numpy(), rtol=1e-10, atol=1e-12)


class TestSequenceParallelBackward:
    """Backward of the sequence-parallel block: LayerNorm's backward against torch
    float64 autograd and finite differences; the whole block's gradients against
    autograd of the unsharded block."""

    def test_dropout_bwd_is_the_adjoint_of_dropout(self):
        # Dropout with a fixed mask is linear in its input, so its backward is the
        # adjoint: dropout_bwd(dY)[k] = <dY, Dropout(e_k)> for every unit input e_k
        rng = np.random.default_rng(74)
        keep = (rng.random((3, 5)) < 0.6).astype(np.uint8)
        dY = rng.standard_normal((3, 5))
        for kp, p in ((keep, 0.7), (None, 1.0)):
            got = seqpar.dropout_bwd(dY, kp, p)
            for idx in np.ndindex(3, 5):
                e = np.zeros((3, 5))
                e[idx] = 1.0
                assert abs(got[idx] - (dY * seqpar.dropout_residual(np.zeros((3, 5)), e, kp, p)).sum()) < 1e-15

    def test_layernorm_bwd_torch(self):
        rng = np.random.default_rng(71)
        X = rng.standard_normal((6, 40)) * 2 + 0.3
        g, b = 1 + 0.1 * rng.standard_normal(40), 0.1 * rng.standard_normal(40)
        dY = rng.standard_normal((6, 40))
        r = seqpar.layernorm_bwd(X, g, dY)
        tX, tg, tb = (torch.tensor(a, requires_grad=True) for a in (X, g, b))
        (torch.nn.functional.layer_norm(tX, (40,), tg, tb, eps=1e-5) * torch.from_numpy(dY)).sum().backward()
        np.testing.assert_allclose(r["dX"], tX.grad.numpy(), rtol=1e-10, atol=1e-12)
        np.testing.assert_allclose(r["dgamma"], tg.grad.numpy(), rtol=1e-10, atol=1e-12)
        np.testing.assert_allclose(r["dbeta"], tb.grad.numpy(), rtol=1e-10, atol=1e-12)

    def test_layernorm_bwd_finite_differences(self):
        rng = np.random.default_rng(72)
        X = rng.standard_normal((3, 8))
        g, b = 1 + 0.2 * rng.standard_normal(8), rng.standard_normal(8)
        dY = rng.standard_normal((3, 8))
        r = seqpar.layernorm_bwd(X, g, dY)
        eps = 1e-6
        for (i, j) in [(0, 0), (1, 5), (2, 7)]:
            Xp, Xm = X.copy(), X.copy()
            Xp[i, j] += eps
            Xm[i, j] -= eps
            num = ((seqpar.layernorm(Xp, g, b) - seqpar.layernorm(Xm, g, b)) * dY).sum() / (2 * eps)
            assert abs(num - r["dX"][i, j]) < 1e-7
        # each row's dX sums to zero (LayerNorm is shift invariant)
        np.testing.assert_allclose(r["dX"].sum(axis=1), 0.0, atol=1e-12)

    @pytest.mark.parametrize("N", [1, 2, 4])
    def test_sp_block_bwd_equals_autograd_of_unsharded_block(self, N):
        s, h, f_full, p = 8, 16, 64, 0.8
        rng = np.random.default_rng(73 + N)
        R = rng.standard_normal((s, h)) + 0.2
        g, b = 1 + 0.1 * rng.standard_normal(h), 0.1 * rng.standard_normal(h)
        A, B = rng.standard_normal((h, f_full)) * 0.2, rng.standard_normal((f_full, h)) * 0.2
        keep = (rng.random((s, h)) < p).astype(np.uint8)
        dRo = rng.standard_normal((s, h))
        shards = [(A[:, j * f_full // N:(j + 1) * f_full // N], B[j * f_full // N:(j + 1) * f_full // N])
                  for j in range(N)]
        got = seqpar.sp_mlp_block_bwd(R, g, b, shards, dRo, keep, p, matched=False)
        tR, tg, tb, tA, tB = (torch.tensor(a, requires_grad=True) for a in (R, g, b, A, B))
        X = torch.nn.functional.layer_norm(tR, (h,), tg, tb, eps=1e-5)
        Z = torch.nn.functional.gelu(X @ tA) @ tB
        out = tR + torch.where(torch.from_numpy(keep) != 0, Z / p, torch.zeros_like(Z))
        (out * torch.from_numpy(dRo)).sum().backward()
        np.testing.assert_allclose(got["dR"], tR.grad.numpy(), rtol=1e-10, atol=1e-12)
        np.testing.assert_allclose(got["dgamma"], tg.grad.numpy(), rtol=1e-10, atol=1e-12)
        np.testing.assert_allclose(got["dbeta"], tb.grad.numpy(), rtol=1e-10, atol=1e-12)
        np.testing.assert_allclose(np.concatenate(got["dA"], axis=1), tA.grad.numpy(), rtol=1e-10, atol=1e-12)
        np.testing.assert_allclose(np.concatenate(got["dB"], axis=0), tB.grad.numpy(), rtol=1e-10, atol=1e-12)
