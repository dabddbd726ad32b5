"""C-ABI checks that need no GPU: the library loads, exports every function the
header declares, and rejects bad arguments on the host before any launch (every
call below fails validation, so no HIP work is ever started)."""
import ctypes as C
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tpshard.h")

tp = pytest.importorskip("attention_shard_math_amd", reason="libtpshard.so not built")
lib = tp.lib

OK, INVALID, UNSUPPORTED, WORKSPACE = 0, 1, 2, 3
P = 0x10000          # a fake, 16-byte aligned "device" pointer: never dereferenced
MIS = 0x10002        # misaligned
# Stream-K area a workspace includes when one of its GEMMs has a tile count (tiles of
# 256 x 192) whose last round fills at most half of the 256-workgroup grid: two
# float32 tile slots per workgroup.
SK_BYTES = 2 * 256 * 256 * 192 * 4


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(tp_[a-z0-9_]+)\s*\(", text)))


def test_every_declared_function_is_exported():
    names = declared_functions()
    assert len(names) >= 12
    for n in names:
        assert hasattr(lib, n), f"{n} declared in tpshard.h but not exported"


def test_status_strings():
    assert lib.tp_status_string(0) == b"TP_OK"
    assert lib.tp_status_string(3) == b"TP_ERR_WORKSPACE"
    assert lib.tp_status_string(99) == b"TP_ERR_UNKNOWN"


def _err():
    return lib.tp_last_error().decode()


class TestValidation:
    def test_column_linear(self):
        f = lib.tp_column_linear
        assert f(7, 4, 8, 8, P, P, None, P, 1, None, 0, None) == INVALID            # dtype
        assert f(1, 4, 8, 8, P, P, None, P, 5, None, 0, None) == INVALID            # activation
        assert f(1, 4, 8, 8, P, P, P, P, 0, None, 0, None) == INVALID               # U_out without act
        assert f(1, -1, 8, 8, P, P, None, P, 1, None, 0, None) == INVALID           # M < 0
        assert f(1, 4, 0, 8, P, P, None, P, 1, None, 0, None) == INVALID            # K == 0
        assert f(1, 4, 12, 8, P, P, None, P, 1, None, 0, None) == UNSUPPORTED       # K % 8
        assert f(1, 4, 8, 20, P, P, None, P, 1, None, 0, None) == UNSUPPORTED       # N % 8
        assert f(1, 4, 8, 8, None, P, None, P, 1, None, 0, None) == INVALID         # X NULL
        assert "X is NULL" in _err()
        assert f(1, 4, 8, 8, P, MIS, None, P, 1, None, 0, None) == UNSUPPORTED      # alignment
        assert f(1, 4, 8, 8, P, P, MIS, P, 1, None, 0, None) == UNSUPPORTED
        assert f(1, 1 << 31, 8, 8, P, P, None, P, 1, None, 0, None) == UNSUPPORTED  # too large

    def test_linear_workspace(self):
        # 4 x 1536 x 8: one tile of 48 k-stages, a nearly empty round: the stream-K area
        assert lib.tp_linear_workspace(1, 4, 1536, 8) == SK_BYTES
        assert lib.tp_linear_workspace(1, 4, 1528, 8) == 0                   # under 48 k-stages: never
        assert lib.tp_linear_workspace(1, 4, 8, 8) == 0
        assert lib.tp_linear_workspace(0, 4, 1536, 8) == 0                   # float32: never
        assert lib.tp_linear_workspace(1, 2048, 12288, 6144) == 0            # 256 tiles: one whole round
        assert lib.tp_linear_workspace(1, 2048, 18432, 9216) == SK_BYTES     # 384 tiles: 1.5 rounds
        assert lib.tp_linear_workspace(1, 4096, 18432, 9216) == 0            # 768 tiles: 3 rounds
        f = lib.tp_column_linear
        # a workspace is optional, but a given one must be large enough
        assert f(1, 4, 1536, 8, P, P, None, P, 1, P, SK_BYTES - 1, None) == WORKSPACE
        assert "workspace" in _err()
        assert f(1, 4, 1536, 8, P, P, None, P, 1, MIS, SK_BYTES, None) == UNSUPPORTED
        r = lib.tp_row_linear
        assert r(1, 4, 1536, 8, P, P, P, P, SK_BYTES - 256, None) == WORKSPACE
        assert lib.tp_mlp_fwd_workspace(1, 2048, 12288, 6144) == 0
        assert lib.tp_mlp_fwd_workspace(1, 2048, 18432, 9216) == SK_BYTES
        assert lib.tp_mlp_fwd_workspace(0, 8, 64, 64) == 0
        m = lib.tp_mlp_fwd
        assert lib.tp_mlp_fwd_workspace(1, 4, 16, 24) == 0                  # under 48 k-stages
        assert m(1, 4, 1536, 1536, P, P, P, None, P, P, P, SK_BYTES - 1, None) == WORKSPACE

    def test_operands_of_two_gib_are_rejected_before_any_launch(self):
        # [131072, 8192] bf16 is exactly 2 GiB: the kernels address operands with 32-bit offsets
        M, K, N = 131072, 8192, 8192
        assert lib.tp_column_linear(1, M, K, N, P, P, None, P, 1, None, 0, None) == UNSUPPORTED
        assert "2 GiB" in _err() and "X" in _err()
        assert lib.tp_row_linear(1, 1024, 8, 1 << 27, P, P, P, None, 0, None) == UNSUPPORTED
        assert "W" in _err()
        assert lib.tp_mlp_fwd(1, 16, 1 << 26, 16, P, P, P, None, P, P, None, 0, None) == UNSUPPORTED
        b = lib.tp_mlp_bwd
        need = lib.tp_mlp_bwd_workspace(M, K, 64)
        assert b(M, K, 64, P, P, P, P, P, P, P, P, P, P, need, None) == UNSUPPORTED
        need = lib.tp_attn_fwd_workspace(1, M, K, 2, 64, )
        assert lib.tp_attn_fwd(1, M, K, 2, 64, 1, P, P, P, P, P, need, None) == UNSUPPORTED
        need = lib.tp_vocab_ce_workspace(16, 8192, 0, 1 << 17)
        assert lib.tp_vocab_ce_partials(16, 8192, 0, 1 << 17, P, P, P, P, P, P, P, need, None) == UNSUPPORTED
        assert "E_i" in _err()

    def test_row_linear_and_mlp_fwd(self):
        assert lib.tp_row_linear(1, 4, 8, 8, P, P, None, None, 0, None) == INVALID
        assert lib.tp_mlp_fwd(1, 4, 16, 24, P, P, P, None, None, P, None, 0, None) == INVALID  # Y_i NULL
        assert lib.tp_mlp_fwd(1, 4, 16, 20, P, P, P, None, P, P, None, 0, None) == UNSUPPORTED

    def test_mlp_bwd(self):
        M, h, f = 32, 1536, 1536
        need = lib.tp_mlp_bwd_workspace(M, h, f)
        # dU, then the stream-K area (these products have fewer tiles than the grid, and
        # dU = dZ B_i^T and dX have 48 k-stages)
        assert need == M * f * 2 + SK_BYTES and need % 256 == 0
        assert lib.tp_mlp_bwd_workspace(3, 8, 8) == 256                     # under 48 k-stages: no area
        # 2048 x 6144 / 6144 x 12288 / 12288 x 6144 / 2048 x 12288 fill whole rounds: no area
        assert lib.tp_mlp_bwd_workspace(2048, 12288, 6144) == 2048 * 6144 * 2
        b = lib.tp_mlp_bwd
        # U_i (or Y_i) NULL selects activation recompute, which needs the larger workspace
        need_re = lib.tp_mlp_bwd_recompute_workspace(M, h, f)
        assert need_re == 3 * M * f * 2 + SK_BYTES
        assert b(M, h, f, P, P, P, None, P, P, P, P, P, P, need, None) == WORKSPACE
        assert b(M, h, f, P, P, P, P, None, P, P, P, P, P, need_re - 1, None) == WORKSPACE
        assert b(M, h, f, P, P, P, None, None, None, P, P, P, P, need_re, None) == INVALID  # dZ NULL
        assert b(M, h, f, P, P, P, MIS, P, P, P, P, P, P, need_re, None) == UNSUPPORTED  # misaligned U_i
        assert b(M, h, f, P, P, P, P, P, P, P, P, P, P, need - 1, None) == WORKSPACE
        assert b(M, h, f, P, P, P, P, P, P, P, P, P, None, need, None) == WORKSPACE
        assert "workspace" in _err()
        assert b(M, h, f, P, P, P, P, P, None, P, P, P, P, need, None) == INVALID      # dZ NULL

    def test_mlp_bwd_noalloc(self):
        cap = lib.tp_mlp_bwd_noalloc_max_bytes()
        assert cap == 80 << 20
        n = lib.tp_mlp_bwd_noalloc
        f = 8192
        M = cap // (2 * f) + 1  # dU one row past the scratch
        assert n(M, 64, f, P, P, P, P, P, P, P, P, P, None) == UNSUPPORTED
        assert "scratch" in _err()
        assert n(64, 64, 128, P, P, P, None, P, P, P, P, P, None) == INVALID     # U_i NULL: no recompute
        assert n(64, 64, 128, P, P, P, P, P, None, P, P, P, None) == INVALID     # dZ NULL
        assert n(64, 64, 124, P, P, P, P, P, P, P, P, P, None) == UNSUPPORTED    # f % 8

    def test_attention(self):
        assert lib.tp_attn_core(1, 16, 2, 96, 1, P, P, None) == UNSUPPORTED  # d_head
        assert lib.tp_attn_core(1, 16, 0, 128, 1, P, P, None) == INVALID
        assert lib.tp_attn_core(-1, 16, 2, 128, 1, P, P, None) == INVALID
        ws = lib.tp_attn_fwd_workspace(2, 100, 256, 3, 64)   # K = 256 and 192: no stream-K area
        assert ws == (2 * 100 * 9 * 64 * 2 + 2 * 100 * 3 * 64 * 2 + (-(2 * 100 * 9 * 64 * 2) % 256)
                      + (-(2 * 100 * 3 * 64 * 2) % 256))
        assert lib.tp_attn_fwd_workspace(1, 100, 2048, 3, 64) == (
            100 * 9 * 64 * 2 + (-(100 * 9 * 64 * 2) % 256) + 100 * 3 * 64 * 2 + (-(100 * 3 * 64 * 2) % 256) + SK_BYTES)
        # the GPT-3 shard's QKV (192 tiles) and Wo (512 tiles) products use no stream-K area
        t, w = 2048, 12 * 128
        assert lib.tp_attn_fwd_workspace(1, 2048, 12288, 12, 128) == t * 3 * w * 2 + t * w * 2
        assert lib.tp_attn_fwd(2, 100, 256, 3, 64, 1, P, P, P, P, P, ws - 16, None) == WORKSPACE
        assert lib.tp_attn_fwd(2, 100, 260, 3, 64, 1, P, P, P, P, P, ws, None) == UNSUPPORTED  # h % 8

    def test_attention_backward(self):
        ws = lib.tp_attn_core_bwd_workspace(2, 100, 3, 128)
        assert ws == 2 * 100 * 3 * 4 + (-(2 * 100 * 3 * 4) % 256)
        cb = lib.tp_attn_core_bwd
        assert cb(1, 16, 2, 96, 1, P, P, P, P, P, P, ws, None) == UNSUPPORTED       # d_head
        assert cb(1, 16, 2, 128, 1, P, P, None, P, P, P, ws, None) == INVALID      # dO NULL
        assert cb(1, 16, 2, 128, 1, P, P, P, None, P, P, ws, None) == INVALID      # lse NULL
        assert cb(1, 16, 2, 128, 1, P, P, P, P, P, P, 16 * 2 * 4 - 4, None) == WORKSPACE
        assert cb(1, 16, 2, 128, 1, P, MIS, P, P, P, P, 256, None) == UNSUPPORTED
        assert cb(0, 16, 2, 128, 1, None, None, None, None, None, None, 0, None) == OK
        # 384-wide heads: rowsum(dO*O), then float32 partial slots of 64 rows x 384 for
        # dQ, dK and dV, 4 chunks per 64-row block, once a walk of 32-row steps is cut
        # into chunks (chunk length max(16, ceil(ceil(s / 32) / 4)) steps)
        s = 4096
        ws384 = lib.tp_attn_core_bwd_workspace(1, s, 6, 384)
        slot_bytes = 6 * (s // 64) * 4 * 64 * 384 * 4
        assert ws384 == 6 * s * 4 + 3 * slot_bytes
        assert lib.tp_attn_core_bwd_workspace(1, 300, 2, 384) == 2 * 300 * 4 + (-(2 * 300 * 4) % 256)  # 10 steps
        assert lib.tp_attn_core_bwd_workspace(1, s, 6, 96) == 0
        assert cb(1, s, 6, 384, 1, P, P, P, P, P, P, ws384 - 1, None) == WORKSPACE
        need = lib.tp_attn_bwd_workspace(1, 64, 256, 2, 64)
        t, w = 64, 128
        assert need == (-(-t * w * 2 // 256) * 256 + -(-t * 3 * w * 2 // 256) * 256
                        + -(-lib.tp_attn_core_bwd_workspace(1, 64, 2, 64) // 256) * 256)  # no product has 48 k-stages
        assert lib.tp_attn_bwd_workspace(1, 64, 2048, 2, 64) == (
            -(-t * w * 2 // 256) * 256 + -(-t * 3 * w * 2 // 256) * 256
            + -(-lib.tp_attn_core_bwd_workspace(1, 64, 2, 64) // 256) * 256 + SK_BYTES)  # dO = dOut Wo^T: K = 2048
        b = lib.tp_attn_bwd
        args = [P] * 10  # X, Wqkv_i, Wo_i, QKV, O, lse, dOut, dX_i, dWqkv_i, dWo_i
        assert b(1, 64, 256, 2, 64, 1, *args, P, need - 1, None) == WORKSPACE
        assert b(1, 64, 260, 2, 64, 1, *args, P, need, None) == UNSUPPORTED           # h % 8
        assert b(1, 64, 256, 2, 64, 1, *args[:9], None, P, need, None) == INVALID  # dWo NULL
        assert b(1, 64, 256, 2, 64, 1, *args[:6], None, *args[7:], P, need, None) == INVALID  # dOut NULL
        f = lib.tp_attn_fwd_train
        assert f(1, 64, 256, 2, 64, 1, P, P, P, P, P, P, None, None) == INVALID     # lse NULL
        assert f(1, 64, 256, 2, 96, 1, P, P, P, P, P, P, P, None) == UNSUPPORTED
        assert f(0, 64, 256, 2, 64, 1, None, None, None, None, None, None, None, None) == OK

    def test_vocab_embed(self):
        e = lib.tp_vocab_embed
        assert e(P, 4, P, 10, 10, 8, P, None) == INVALID   # lo == hi
        assert e(P, 4, P, -1, 10, 8, P, None) == INVALID   # lo < 0
        assert e(P, -4, P, 0, 10, 8, P, None) == INVALID
        assert e(P, 4, P, 0, 10, 12, P, None) == UNSUPPORTED
        assert e(None, 4, P, 0, 10, 8, P, None) == INVALID
        assert e(P, 4, P, 0, 10, 8, MIS, None) == UNSUPPORTED

    def test_vocab_ce(self):
        # per row, 8 bytes for each 48-column slot (four per 192-column tile), rounded
        # up to 256 bytes, then the stream-K area when the logits GEMM uses one
        M, h, lo, hi = 16, 64, 40, 104
        need = lib.tp_vocab_ce_workspace(M, h, lo, hi)
        assert need == 512 and need % 256 == 0                        # 16 rows x 4 slots; h = 64: no stream-K
        assert lib.tp_vocab_ce_workspace(3, 64, 0, 8) == 256
        assert lib.tp_vocab_ce_workspace(16, 2048, lo, hi) == 512 + SK_BYTES
        assert lib.tp_vocab_ce_workspace(2048, 12288, 0, 6144) == 2048 * 128 * 8  # 256 tiles: no area
        assert lib.tp_vocab_ce_workspace(2048, 12288, 0, 6288) == 2048 * 132 * 8 + SK_BYTES  # 264 tiles
        assert lib.tp_vocab_ce_workspace(3, 64, 8, 8) == 0
        assert lib.tp_vocab_ce_workspace(3, 0, 0, 8) == 0
        c = lib.tp_vocab_ce_partials
        a7 = [P] * 7  # H, E_i, targets, rowmax_i, sumexp_i, tlogit_i, ws
        assert c(M, h, 10, 10, *a7, need, None) == INVALID          # lo == hi
        assert c(M, h, -8, 8, *a7, need, None) == INVALID          # lo < 0
        assert c(-1, h, lo, hi, *a7, need, None) == INVALID
        assert c(M, h, 0, 12, *a7, need, None) == UNSUPPORTED      # slice % 8
        assert c(M, 20, lo, hi, *a7, need, None) == UNSUPPORTED    # h % 8
        assert c(M, h, lo, hi, P, P, None, P, P, P, P, need, None) == INVALID      # targets NULL
        assert c(M, h, lo, hi, None, P, P, P, P, P, P, need, None) == INVALID
        assert c(M, h, lo, hi, P, MIS, P, P, P, P, P, need, None) == UNSUPPORTED
        assert c(M, h, lo, hi, P, P, P, None, P, P, P, need, None) == INVALID      # rowmax_i NULL
        assert "rowmax_i" in _err()
        assert c(M, h, lo, hi, *a7, need - 1, None) == WORKSPACE
        assert c(M, h, lo, hi, P, P, P, P, P, P, None, need, None) == WORKSPACE
        assert "workspace" in _err()
        assert c(0, h, lo, hi, None, None, None, None, None, None, None, 0, None) == OK  # empty
        arr = (C.c_void_p * 17)(*([P] * 17))
        loss = lib.tp_vocab_ce_loss
        assert loss(M, arr, arr, arr, 0, P, P, None) == INVALID
        assert loss(M, arr, arr, arr, 17, P, P, None) == INVALID
        assert loss(-1, arr, arr, arr, 2, P, P, None) == INVALID
        assert loss(M, None, arr, arr, 2, P, P, None) == INVALID
        assert loss(M, arr, None, arr, 2, P, P, None) == INVALID
        assert loss(M, arr, arr, arr, 2, P, None, None) == INVALID                 # loss_sum NULL
        assert loss(M, arr, arr, arr, 2, None, P, None) == INVALID                 # loss_rows NULL
        bad = (C.c_void_p * 2)(P, None)
        assert loss(M, arr, arr, bad, 2, P, P, None) == INVALID
        assert "tlogit_parts" in _err()
        assert loss(M, bad, arr, arr, 2, P, P, None) == INVALID
        assert "rowmax_parts" in _err()

    def test_sequence_parallel(self):
        ln = lib.tp_layernorm
        assert ln(-1, 64, P, P, P, 1e-5, P, None) == INVALID
        assert ln(4, 0, P, P, P, 1e-5, P, None) == INVALID
        assert ln(4, 60, P, P, P, 1e-5, P, None) == UNSUPPORTED           # h % 8
        assert ln(4, 32776, P, P, P, 1e-5, P, None) == UNSUPPORTED        # h too large
        assert ln(4, 64, P, P, P, -1.0, P, None) == INVALID               # eps < 0
        assert ln(4, 64, P, None, P, 1e-5, P, None) == INVALID            # gamma NULL
        assert ln(4, 64, P, P, P, 1e-5, MIS, None) == UNSUPPORTED
        assert ln(0, 64, None, None, None, 1e-5, None, None) == OK        # empty
        arr = (C.c_void_p * 17)(*([P] * 17))
        ag = lib.tp_sp_all_gather
        assert ag(0, arr, 4, 64, P, None) == INVALID
        assert ag(17, arr, 4, 64, P, None) == INVALID
        assert ag(2, arr, 4, 12, P, None) == UNSUPPORTED
        assert ag(2, arr, -1, 64, P, None) == INVALID
        assert ag(2, (C.c_void_p * 2)(P, MIS), 4, 64, P, None) == UNSUPPORTED
        assert "slices[1]" in _err()
        assert ag(2, None, 0, 64, None, None) == OK
        rs = lib.tp_sp_reduce_scatter
        assert rs(4, arr, 18, 64, 0, P, None, 1.0, P, None) == INVALID     # s % n
        assert rs(4, arr, 16, 64, 4, P, None, 1.0, P, None) == INVALID     # rank
        assert rs(4, arr, 16, 64, -1, P, None, 1.0, P, None) == INVALID
        assert rs(4, arr, 16, 64, 0, P, P, 0.0, P, None) == INVALID        # keep_prob
        assert rs(4, arr, 16, 64, 0, P, P, 1.5, P, None) == INVALID
        assert rs(4, arr, 16, 64, 0, P, P + 2, 0.5, P, None) == UNSUPPORTED  # keep alignment
        assert rs(4, arr, 16, 64, 0, MIS, None, 1.0, P, None) == UNSUPPORTED  # residual misaligned
        assert rs(4, arr, 16, 64, 0, None, None, 1.0, None, None) == INVALID  # out NULL
        assert rs(4, arr, 16, 20, 0, P, None, 1.0, P, None) == UNSUPPORTED
        assert rs(2, (C.c_void_p * 2)(P, None), 16, 64, 0, P, None, 1.0, P, None) == INVALID
        assert rs(17, arr, 17, 64, 0, P, None, 1.0, P, None) == INVALID
        assert rs(4, None, 0, 64, 0, None, None, 1.0, None, None) == OK

    def test_sequence_parallel_backward(self):
        need = lib.tp_layernorm_bwd_workspace(10, 64)
        assert need >= 10 * 8 and need % 4 == 0
        lb = lib.tp_layernorm_bwd
        assert lb(-1, 64, P, P, P, None, 1e-5, P, P, P, P, need, None) == INVALID
        assert lb(10, 60, P, P, P, None, 1e-5, P, P, P, P, need, None) == UNSUPPORTED      # h % 8
        assert lb(10, 24584, P, P, P, None, 1e-5, P, P, P, P, need, None) == UNSUPPORTED   # h too large
        assert lb(10, 64, P, P, P, None, -1.0, P, P, P, P, need, None) == INVALID           # eps
        assert lb(10, 64, P, P, None, None, 1e-5, P, P, P, P, need, None) == INVALID        # dY NULL
        assert lb(10, 64, P, P, P, MIS, 1e-5, P, P, P, P, need, None) == UNSUPPORTED        # dRes misaligned
        assert lb(10, 64, P, P, P, None, 1e-5, P, None, P, P, need, None) == INVALID        # dgamma NULL
        assert lb(10, 64, P, P, P, None, 1e-5, P, P, P, P, need - 1, None) == WORKSPACE
        assert lb(10, 64, P, P, P, None, 1e-5, P, P, P, None, need, None) == WORKSPACE
        db = lib.tp_sp_dropout_bwd
        assert db(-1, 64, P, None, 1.0, P, None) == INVALID
        assert db(4, 12, P, None, 1.0, P, None) == UNSUPPORTED
        assert db(4, 64, P, P, 0.0, P, None) == INVALID
        assert db(4, 64, P, P + 2, 0.5, P, None) == UNSUPPORTED
        assert db(4, 64, None, None, 1.0, P, None) == INVALID
        assert db(4, 64, P, None, 1.0, MIS, None) == UNSUPPORTED
        assert db(0, 64, None, None, 1.0, None, None) == OK

    def test_shard_sum(self):
        arr = (C.c_void_p * 17)(*([P] * 17))
        s = lib.tp_shard_sum
        assert s(0, arr, 0, 16, P, None) == INVALID
        assert s(0, arr, 17, 16, P, None) == INVALID
        assert s(0, arr, 4, -1, P, None) == INVALID
        assert s(0, None, 4, 0, None, None) == OK  # empty: nothing to touch
        assert s(5, arr, 4, 16, P, None) == INVALID
        bad = (C.c_void_p * 2)(P, None)
        assert s(0, bad, 2, 16, P, None) == INVALID
        mis = (C.c_void_p * 2)(P, MIS)
        assert s(0, mis, 2, 16, P, None) == UNSUPPORTED
        assert "partials[1]" in _err()
