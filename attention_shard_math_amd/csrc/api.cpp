// C-ABI entry points of libtpshard: argument validation on the host, then kernel
// launches on the caller's stream. No allocation, no synchronisation, no
// exceptions across the interface. The operations and their citations are
// documented in include/tpshard.h.
#include <initializer_list>
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>

#include "attn.hpp"
#include "vocab_ce.hpp"
#include "seqpar.hpp"
#include "bandwidth.hpp"
#include "gemm_bf16.hpp"
#include "gemm_f32.hpp"
#include "api_internal.hpp"
#include "tpshard.h"

#define TP_API extern "C" __attribute__((visibility("default")))

namespace {

thread_local std::string g_last_error;

tp_status fail(tp_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

tp_status ok() {
  g_last_error.clear();
  return TP_OK;
}

tp_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(TP_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

constexpr int64_t kMaxDim = (int64_t(1) << 31) - 1;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Validation helpers return TP_OK or an error (with the message set).
tp_status check_dims(const char* fn, int64_t M, int64_t K, int64_t N) {
  if (M < 0 || K <= 0 || N <= 0)
    return fail(TP_ERR_INVALID_ARG, "%s: sizes must satisfy M >= 0, K > 0, N > 0 (got M=%lld K=%lld N=%lld)", fn,
                (long long)M, (long long)K, (long long)N);
  if (M > kMaxDim || K > kMaxDim || N > kMaxDim)
    return fail(TP_ERR_UNSUPPORTED, "%s: a dimension exceeds 2^31-1", fn);
  if (K % 8 || N % 8)
    return fail(TP_ERR_UNSUPPORTED, "%s: K and N must be multiples of 8 (got K=%lld N=%lld)", fn, (long long)K,
                (long long)N);
  return TP_OK;
}

tp_status check_ptr(const char* fn, const char* name, const void* p) {
  if (!p) return fail(TP_ERR_INVALID_ARG, "%s: %s is NULL", fn, name);
  if (!aligned16(p)) return fail(TP_ERR_UNSUPPORTED, "%s: %s is not 16-byte aligned", fn, name);
  return TP_OK;
}

tp_status check_opt_ptr(const char* fn, const char* name, const void* p) {
  if (p && !aligned16(p)) return fail(TP_ERR_UNSUPPORTED, "%s: %s is not 16-byte aligned", fn, name);
  return TP_OK;
}

// The GEMM and attention kernels address each operand through a buffer resource
// with 32-bit byte offsets, so no operand may reach 2 GiB.
constexpr double kMaxOperandBytes = 2147483632.0;  // 2^31 - 16
tp_status check_bytes(const char* fn, const char* name, int64_t rows, int64_t cols, int64_t elem) {
  if ((double)rows * (double)cols * (double)elem >= kMaxOperandBytes)
    return fail(TP_ERR_UNSUPPORTED, "%s: %s [%lld x %lld] reaches 2 GiB; the kernels address operands with 32-bit byte offsets",
                fn, name, (long long)rows, (long long)cols);
  return TP_OK;
}

#define TRY(expr)                      \
  do {                                 \
    const tp_status _s = (expr);       \
    if (_s != TP_OK) return _s;        \
  } while (0)

size_t round256(size_t x) { return (x + 255) & ~size_t(255); }

// Stream-K area of a bf16 GEMM (0 when its tiles fill whole rounds of the grid).
size_t sk_need(int64_t M, int64_t N, int64_t K) {
  if (M <= 0 || N <= 0 || K <= 0 || M > kMaxDim || N > kMaxDim || K > kMaxDim) return 0;
  return tps::gemm_bf16_sk_workspace((int)M, (int)N, (int)K);
}
size_t sk_max(std::initializer_list<size_t> v) {
  size_t m = 0;
  for (size_t x : v) m = x > m ? x : m;
  return m;
}

tps::GemmArgs make_args(const void* A, int64_t lda, const void* B, int64_t ldb, int64_t M, int64_t N, int64_t K,
                        void* C, int64_t ldc) {
  tps::GemmArgs g{};
  g.A = static_cast<const uint16_t*>(A);
  g.B = static_cast<const uint16_t*>(B);
  g.lda = lda;
  g.ldb = ldb;
  g.M = (int)M;
  g.N = (int)N;
  g.K = (int)K;
  g.C = C;
  g.ldc = ldc;
  return g;
}

hipStream_t as_stream(void* s) { return static_cast<hipStream_t>(s); }

}  // namespace

TP_API const char* tp_status_string(tp_status s) {
  switch (s) {
    case TP_OK: return "TP_OK";
    case TP_ERR_INVALID_ARG: return "TP_ERR_INVALID_ARG";
    case TP_ERR_UNSUPPORTED: return "TP_ERR_UNSUPPORTED";
    case TP_ERR_WORKSPACE: return "TP_ERR_WORKSPACE";
    case TP_ERR_HIP: return "TP_ERR_HIP";
  }
  return "TP_ERR_UNKNOWN";
}

TP_API const char* tp_last_error(void) { return g_last_error.c_str(); }

namespace {
// Workspace of an optional stream-K area passed to a call that takes one: NULL
// runs the products one tile per workgroup; a non-NULL workspace must hold `need`.
tp_status check_opt_ws(const char* fn, const void* ws, size_t ws_bytes, size_t need) {
  if (ws && ws_bytes < need)
    return fail(TP_ERR_WORKSPACE, "%s: workspace of %zu bytes required, got %zu", fn, need, ws_bytes);
  return check_opt_ptr(fn, "ws", ws);
}
}  // namespace

TP_API size_t tp_linear_workspace(tp_dtype dt, int64_t M, int64_t K, int64_t N) {
  return dt == TP_BF16 ? sk_need(M, N, K) : 0;
}

TP_API tp_status tp_column_linear(tp_dtype dt, int64_t M, int64_t K, int64_t N, const void* X, const void* W,
                                  void* U_out, void* Y_out, int act, void* ws, size_t ws_bytes, void* stream) {
  const char* fn = "tp_column_linear";
  if (dt != TP_F32 && dt != TP_BF16) return fail(TP_ERR_INVALID_ARG, "%s: unknown dtype %d", fn, (int)dt);
  if (act != TP_ACT_NONE && act != TP_ACT_GELU) return fail(TP_ERR_INVALID_ARG, "%s: unknown activation %d", fn, act);
  if (act == TP_ACT_NONE && U_out)
    return fail(TP_ERR_INVALID_ARG, "%s: U_out must be NULL without an activation", fn);
  TRY(check_dims(fn, M, K, N));
  if (M == 0) return ok();  // nothing to compute; empty tensors may carry NULL
  TRY(check_ptr(fn, "X", X));
  TRY(check_ptr(fn, "W", W));
  TRY(check_ptr(fn, "Y_out", Y_out));
  TRY(check_opt_ptr(fn, "U_out", U_out));
  TRY(check_opt_ws(fn, ws, ws_bytes, tp_linear_workspace(dt, M, K, N)));
  if (dt == TP_F32)
    return hip_status(tps::gemm_f32(static_cast<const float*>(X), static_cast<const float*>(W), (int)M, (int)N, (int)K,
                                    static_cast<float*>(Y_out), static_cast<float*>(U_out), act == TP_ACT_GELU,
                                    as_stream(stream)),
                      fn);
  TRY(check_bytes(fn, "X", M, K, 2));
  TRY(check_bytes(fn, "W", K, N, 2));
  tps::GemmArgs g = make_args(X, K, W, N, M, N, K, Y_out, N);
  g.U = static_cast<uint16_t*>(U_out);
  g.ldu = N;
  tps::gemm_bf16_sk_attach(g, ws);
  return hip_status(tps::gemm_bf16(g, true, false, act == TP_ACT_GELU ? tps::EPI_GELU : tps::EPI_BF16,
                                   as_stream(stream)),
                    fn);
}

TP_API tp_status tp_row_linear(tp_dtype dt, int64_t M, int64_t K, int64_t N, const void* Y, const void* W,
                               float* Z_out, void* ws, size_t ws_bytes, void* stream) {
  const char* fn = "tp_row_linear";
  if (dt != TP_F32 && dt != TP_BF16) return fail(TP_ERR_INVALID_ARG, "%s: unknown dtype %d", fn, (int)dt);
  TRY(check_dims(fn, M, K, N));
  if (M == 0) return ok();
  TRY(check_ptr(fn, "Y", Y));
  TRY(check_ptr(fn, "W", W));
  TRY(check_ptr(fn, "Z_out", Z_out));
  TRY(check_opt_ws(fn, ws, ws_bytes, tp_linear_workspace(dt, M, K, N)));
  if (dt == TP_F32)
    return hip_status(tps::gemm_f32(static_cast<const float*>(Y), static_cast<const float*>(W), (int)M, (int)N, (int)K,
                                    Z_out, nullptr, false, as_stream(stream)),
                      fn);
  TRY(check_bytes(fn, "Y", M, K, 2));
  TRY(check_bytes(fn, "W", K, N, 2));
  tps::GemmArgs g = make_args(Y, K, W, N, M, N, K, Z_out, N);
  tps::gemm_bf16_sk_attach(g, ws);
  return hip_status(tps::gemm_bf16(g, true, false, tps::EPI_F32, as_stream(stream)), fn);
}

TP_API size_t tp_mlp_fwd_workspace(tp_dtype dt, int64_t M, int64_t h, int64_t f) {
  // the two products run one after the other and share the area
  return sk_max({tp_linear_workspace(dt, M, h, f), tp_linear_workspace(dt, M, f, h)});
}

TP_API tp_status tp_mlp_fwd(tp_dtype dt, int64_t M, int64_t h, int64_t f, const void* X, const void* A_i,
                            const void* B_i, void* U_i, void* Y_i, float* Z_i, void* ws, size_t ws_bytes,
                            void* stream) {
  const char* fn = "tp_mlp_fwd";
  if (dt != TP_F32 && dt != TP_BF16) return fail(TP_ERR_INVALID_ARG, "%s: unknown dtype %d", fn, (int)dt);
  TRY(check_dims(fn, M, h, f));
  if (M == 0) return ok();
  TRY(check_ptr(fn, "X", X));
  TRY(check_ptr(fn, "A_i", A_i));
  TRY(check_ptr(fn, "B_i", B_i));
  TRY(check_ptr(fn, "Y_i", Y_i));
  TRY(check_ptr(fn, "Z_i", Z_i));
  TRY(check_opt_ptr(fn, "U_i", U_i));
  TRY(check_opt_ws(fn, ws, ws_bytes, tp_mlp_fwd_workspace(dt, M, h, f)));
  if (dt == TP_BF16) {  // validate both products before the first launch
    TRY(check_bytes(fn, "X", M, h, 2));
    TRY(check_bytes(fn, "A_i", h, f, 2));
    TRY(check_bytes(fn, "Y_i", M, f, 2));
    TRY(check_bytes(fn, "B_i", f, h, 2));
  }
  TRY(tp_column_linear(dt, M, h, f, X, A_i, U_i, Y_i, TP_ACT_GELU, ws, ws_bytes, stream));
  return tp_row_linear(dt, M, f, h, Y_i, B_i, Z_i, ws, ws_bytes, stream);
}

namespace {
// Stream-K area shared by the four backward GEMMs (they run one after another).
size_t mlp_bwd_sk(int64_t M, int64_t h, int64_t f) {
  return sk_max({sk_need(M, f, h), sk_need(f, h, M), sk_need(h, f, M), sk_need(M, h, f)});
}
}  // namespace

TP_API size_t tp_mlp_bwd_workspace(int64_t M, int64_t h, int64_t f) {
  if (M < 0 || f < 0) return 0;
  return round256((size_t)M * (size_t)f * 2) + mlp_bwd_sk(M, h, f);
}

TP_API size_t tp_mlp_bwd_recompute_workspace(int64_t M, int64_t h, int64_t f) {
  if (M < 0 || f < 0) return 0;
  return 3 * round256((size_t)M * (size_t)f * 2) + mlp_bwd_sk(M, h, f);
}

namespace tps {

tp_status api_fail(tp_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

tp_status api_ok() { return ok(); }

tp_status mlp_bwd_validate(const char* fn, int64_t M, int64_t h, int64_t f, const void* X, const void* A_i,
                           const void* B_i, const void* U_i, const void* Y_i, const void* dZ, const float* dX_i,
                           const float* dA_i, const float* dB_i) {
  TRY(check_dims(fn, M, h, f));
  TRY(check_opt_ptr(fn, "dA_i", dA_i));
  TRY(check_opt_ptr(fn, "dB_i", dB_i));
  if (M > 0) {  // with M == 0 only the (zero) weight gradients are written
    TRY(check_ptr(fn, "X", X));
    TRY(check_ptr(fn, "A_i", A_i));
    TRY(check_ptr(fn, "B_i", B_i));
    TRY(check_opt_ptr(fn, "U_i", U_i));
    TRY(check_opt_ptr(fn, "Y_i", Y_i));
    TRY(check_ptr(fn, "dZ", dZ));
    TRY(check_opt_ptr(fn, "dX_i", dX_i));
    TRY(check_bytes(fn, "X", M, h, 2));
    TRY(check_bytes(fn, "dZ", M, h, 2));
    TRY(check_bytes(fn, "A_i", h, f, 2));
    TRY(check_bytes(fn, "B_i", f, h, 2));
    TRY(check_bytes(fn, "U_i", M, f, 2));
  }
  return TP_OK;
}

tp_status mlp_bwd_products(const char* fn, int64_t M, int64_t h, int64_t f, const void* X, const void* A_i,
                           const void* B_i, const void* U_i, const void* Y_i, const void* dZ, float* dX_i,
                           float* dA_i, float* dB_i, uint16_t* dU, void* sk, hipStream_t s) {
  if (M > 0) {
    // dU = (dZ B_i^T) * GeLU'(U_i): A = dZ [M,h] (K-contig), B(k,n) = B_i[n, k] (K-contig).
    tps::GemmArgs g = make_args(dZ, h, B_i, h, M, f, h, dU, f);
    g.Uin = static_cast<const uint16_t*>(U_i);
    g.ldu = f;
    tps::gemm_bf16_sk_attach(g, sk);
    TRY(hip_status(tps::gemm_bf16(g, true, true, tps::EPI_DGELU, s), fn));
  }
  if (dB_i) {  // dB = Y^T dZ: A(m,k) = Y[k, m] (M-contig), B(k,n) = dZ[k, n] (N-contig)
    tps::GemmArgs g = make_args(Y_i, f, dZ, h, f, h, M, dB_i, h);
    tps::gemm_bf16_sk_attach(g, sk);
    TRY(hip_status(tps::gemm_bf16(g, false, false, tps::EPI_F32, s), fn));
  }
  if (dA_i) {  // dA = X^T dU: A(m,k) = X[k, m], B(k,n) = dU[k, n]
    tps::GemmArgs g = make_args(X, h, dU, f, h, f, M, dA_i, f);
    tps::gemm_bf16_sk_attach(g, sk);
    TRY(hip_status(tps::gemm_bf16(g, false, false, tps::EPI_F32, s), fn));
  }
  if (dX_i && M > 0) {  // dX = dU A_i^T: A = dU [M,f] (K-contig), B(k,n) = A_i[n, k] (K-contig)
    tps::GemmArgs g = make_args(dU, f, A_i, f, M, h, f, dX_i, h);
    tps::gemm_bf16_sk_attach(g, sk);
    TRY(hip_status(tps::gemm_bf16(g, true, true, tps::EPI_F32, s), fn));
  }
  return ok();
}

}  // namespace tps

TP_API tp_status tp_mlp_bwd(int64_t M, int64_t h, int64_t f, const void* X, const void* A_i, const void* B_i,
                            const void* U_i, const void* Y_i, const void* dZ, float* dX_i, float* dA_i, float* dB_i,
                            void* ws, size_t ws_bytes, void* stream) {
  const char* fn = "tp_mlp_bwd";
  TRY(tps::mlp_bwd_validate(fn, M, h, f, X, A_i, B_i, U_i, Y_i, dZ, dX_i, dA_i, dB_i));
  // Without a saved U_i or Y_i the column GEMM + GeLU is recomputed into the
  // workspace, with the forward's kernel, so the bits equal the forward's.
  const bool recompute = M > 0 && (!U_i || !Y_i);
  const size_t need = recompute ? tp_mlp_bwd_recompute_workspace(M, h, f) : tp_mlp_bwd_workspace(M, h, f);
  if (need && (!ws || ws_bytes < need))
    return fail(TP_ERR_WORKSPACE, "%s: workspace of %zu bytes required, got %zu%s", fn, need, ws_bytes,
                ws ? "" : " (NULL)");
  TRY(check_opt_ptr(fn, "ws", ws));
  uint16_t* dU = static_cast<uint16_t*>(ws);
  // the stream-K area follows the activations
  void* sk = mlp_bwd_sk(M, h, f) ? static_cast<char*>(ws) + (recompute ? 3 : 1) * round256((size_t)M * (size_t)f * 2)
                                 : nullptr;
  if (recompute) {
    const size_t act = round256((size_t)M * (size_t)f * 2);
    uint16_t* U_re = reinterpret_cast<uint16_t*>(static_cast<char*>(ws) + act);
    uint16_t* Y_re = reinterpret_cast<uint16_t*>(static_cast<char*>(ws) + 2 * act);
    TRY(tp_column_linear(TP_BF16, M, h, f, X, A_i, U_re, Y_re, TP_ACT_GELU, nullptr, 0, stream));
    if (!U_i) U_i = U_re;
    if (!Y_i) Y_i = Y_re;
  }
  return tps::mlp_bwd_products(fn, M, h, f, X, A_i, B_i, U_i, Y_i, dZ, dX_i, dA_i, dB_i, dU, sk, as_stream(stream));
}

namespace {
tp_status check_attn_shape(const char* fn, int64_t b, int64_t s, int64_t Hl, int64_t d) {
  if (b < 0 || s < 0 || Hl <= 0 || d <= 0)
    return fail(TP_ERR_INVALID_ARG, "%s: need b >= 0, s >= 0, n_heads_local > 0, d_head > 0", fn);
  if (d != 64 && d != 128 && d != 384)
    return fail(TP_ERR_UNSUPPORTED, "%s: d_head must be 64, 128 or 384 (got %lld)", fn, (long long)d);
  if (b * s > kMaxDim || 3 * Hl * d > kMaxDim || b * Hl * ((s + 127) / 128) > kMaxDim)
    return fail(TP_ERR_UNSUPPORTED, "%s: problem too large", fn);
  // The kernel addresses one sequence's K and V rows with 32-bit byte offsets.
  if ((s + 128) * 3 * Hl * d * 2 >= (int64_t)1 << 31)
    return fail(TP_ERR_UNSUPPORTED, "%s: s * 3 * n_heads_local * d_head too large for one sequence", fn);
  return TP_OK;
}

// Byte checks of the attention shard's GEMM operands (M tokens, w = Hl * d).
tp_status check_attn_bytes(const char* fn, int64_t M, int64_t h, int64_t w) {
  TRY(check_bytes(fn, "X", M, h, 2));
  TRY(check_bytes(fn, "Wqkv_i", h, 3 * w, 2));
  TRY(check_bytes(fn, "QKV", M, 3 * w, 2));
  TRY(check_bytes(fn, "Wo_i", w, h, 2));
  return TP_OK;
}
}  // namespace

TP_API tp_status tp_attn_core(int64_t b, int64_t s, int64_t n_heads_local, int64_t d_head, int causal,
                              const void* QKV, void* O, void* stream) {
  const char* fn = "tp_attn_core";
  TRY(check_attn_shape(fn, b, s, n_heads_local, d_head));
  if (b * s == 0) return ok();
  TRY(check_ptr(fn, "QKV", QKV));
  TRY(check_ptr(fn, "O", O));
  return hip_status(tps::attn_fwd(static_cast<const uint16_t*>(QKV), static_cast<uint16_t*>(O), (int)b, (int)s,
                                  (int)n_heads_local, (int)d_head, causal != 0, as_stream(stream)),
                    fn);
}

TP_API tp_status tp_attn_core_train(int64_t b, int64_t s, int64_t n_heads_local, int64_t d_head, int causal,
                                    const void* QKV, void* O, float* lse, void* stream) {
  const char* fn = "tp_attn_core_train";
  TRY(check_attn_shape(fn, b, s, n_heads_local, d_head));
  if (b * s == 0) return ok();
  TRY(check_ptr(fn, "QKV", QKV));
  TRY(check_ptr(fn, "O", O));
  TRY(check_ptr(fn, "lse", lse));
  return hip_status(tps::attn_fwd(static_cast<const uint16_t*>(QKV), static_cast<uint16_t*>(O), (int)b, (int)s,
                                  (int)n_heads_local, (int)d_head, causal != 0, as_stream(stream), lse),
                    fn);
}

namespace {
// Stream-K area of the attention forward's QKV and Wo GEMMs (they run one after
// the other and share it).
size_t attn_fwd_sk(int64_t M, int64_t h, int64_t w) { return sk_max({sk_need(M, 3 * w, h), sk_need(M, h, w)}); }
}  // namespace

TP_API size_t tp_attn_fwd_workspace(int64_t b, int64_t s, int64_t h, int64_t n_heads_local, int64_t d_head) {
  if (b < 0 || s < 0 || h < 0 || n_heads_local < 0 || d_head < 0) return 0;
  const size_t t = (size_t)b * (size_t)s, w = (size_t)n_heads_local * (size_t)d_head;
  return round256(t * 3 * w * 2) + round256(t * w * 2) + attn_fwd_sk(b * s, h, n_heads_local * d_head);
}

TP_API tp_status tp_attn_fwd(int64_t b, int64_t s, int64_t h, int64_t n_heads_local, int64_t d_head, int causal,
                             const void* X, const void* Wqkv_i, const void* Wo_i, float* out_partial, void* ws,
                             size_t ws_bytes, void* stream) {
  const char* fn = "tp_attn_fwd";
  TRY(check_attn_shape(fn, b, s, n_heads_local, d_head));
  TRY(check_dims(fn, b * s, h, 3 * n_heads_local * d_head));
  if (b * s == 0) return ok();
  TRY(check_ptr(fn, "X", X));
  TRY(check_ptr(fn, "Wqkv_i", Wqkv_i));
  TRY(check_ptr(fn, "Wo_i", Wo_i));
  TRY(check_ptr(fn, "out_partial", out_partial));
  TRY(check_attn_bytes(fn, b * s, h, n_heads_local * d_head));
  const size_t need = tp_attn_fwd_workspace(b, s, h, n_heads_local, d_head);
  if (need && (!ws || ws_bytes < need))
    return fail(TP_ERR_WORKSPACE, "%s: workspace of %zu bytes required, got %zu%s", fn, need, ws_bytes,
                ws ? "" : " (NULL)");
  TRY(check_opt_ptr(fn, "ws", ws));
  const int64_t M = b * s, w = n_heads_local * d_head;
  hipStream_t st = as_stream(stream);
  uint16_t* qkv = static_cast<uint16_t*>(ws);
  uint16_t* O = reinterpret_cast<uint16_t*>(static_cast<char*>(ws) + round256((size_t)M * 3 * w * 2));
  void* sk = static_cast<char*>(ws) + round256((size_t)M * 3 * w * 2) + round256((size_t)M * w * 2);
  {
    tps::GemmArgs g = make_args(X, h, Wqkv_i, 3 * w, M, 3 * w, h, qkv, 3 * w);
    tps::gemm_bf16_sk_attach(g, sk);
    TRY(hip_status(tps::gemm_bf16(g, true, false, tps::EPI_BF16, st), fn));
  }
  TRY(hip_status(tps::attn_fwd(qkv, O, (int)b, (int)s, (int)n_heads_local, (int)d_head, causal != 0, st), fn));
  {
    tps::GemmArgs g = make_args(O, w, Wo_i, h, M, h, w, out_partial, h);
    tps::gemm_bf16_sk_attach(g, sk);
    TRY(hip_status(tps::gemm_bf16(g, true, false, tps::EPI_F32, st), fn));
  }
  return ok();
}

TP_API tp_status tp_attn_fwd_train(int64_t b, int64_t s, int64_t h, int64_t n_heads_local, int64_t d_head,
                                   int causal, const void* X, const void* Wqkv_i, const void* Wo_i,
                                   float* out_partial, void* QKV, void* O, float* lse, void* stream) {
  const char* fn = "tp_attn_fwd_train";
  TRY(check_attn_shape(fn, b, s, n_heads_local, d_head));
  TRY(check_dims(fn, b * s, h, 3 * n_heads_local * d_head));
  if (b * s == 0) return ok();
  TRY(check_ptr(fn, "X", X));
  TRY(check_ptr(fn, "Wqkv_i", Wqkv_i));
  TRY(check_ptr(fn, "Wo_i", Wo_i));
  TRY(check_ptr(fn, "out_partial", out_partial));
  TRY(check_ptr(fn, "QKV", QKV));
  TRY(check_ptr(fn, "O", O));
  TRY(check_ptr(fn, "lse", lse));
  TRY(check_attn_bytes(fn, b * s, h, n_heads_local * d_head));
  const int64_t M = b * s, w = n_heads_local * d_head;
  hipStream_t st = as_stream(stream);
  {
    tps::GemmArgs g = make_args(X, h, Wqkv_i, 3 * w, M, 3 * w, h, QKV, 3 * w);
    TRY(hip_status(tps::gemm_bf16(g, true, false, tps::EPI_BF16, st), fn));
  }
  TRY(hip_status(tps::attn_fwd(static_cast<const uint16_t*>(QKV), static_cast<uint16_t*>(O), (int)b, (int)s,
                               (int)n_heads_local, (int)d_head, causal != 0, st, lse),
                 fn));
  {
    tps::GemmArgs g = make_args(O, w, Wo_i, h, M, h, w, out_partial, h);
    TRY(hip_status(tps::gemm_bf16(g, true, false, tps::EPI_F32, st), fn));
  }
  return ok();
}

TP_API size_t tp_attn_core_bwd_workspace(int64_t b, int64_t s, int64_t n_heads_local, int64_t d_head) {
  if (b <= 0 || s <= 0 || n_heads_local <= 0) return 0;
  if (b * s > kMaxDim || n_heads_local > kMaxDim) return 0;
  if (d_head != 64 && d_head != 128 && d_head != 384) return 0;
  // the 64- and 128-wide kernels share one layout, sized for 128
  return tps::attn_bwd_workspace((int)b, (int)s, (int)n_heads_local, d_head == 384 ? 384 : 128);
}

TP_API tp_status tp_attn_core_bwd(int64_t b, int64_t s, int64_t n_heads_local, int64_t d_head, int causal,
                                  const void* QKV, const void* O, const void* dO, const float* lse, void* dQKV,
                                  void* ws, size_t ws_bytes, void* stream) {
  const char* fn = "tp_attn_core_bwd";
  TRY(check_attn_shape(fn, b, s, n_heads_local, d_head));
  if (b * s == 0) return ok();
  TRY(check_ptr(fn, "QKV", QKV));
  TRY(check_ptr(fn, "O", O));
  TRY(check_ptr(fn, "dO", dO));
  TRY(check_ptr(fn, "lse", lse));
  TRY(check_ptr(fn, "dQKV", dQKV));
  const size_t need = tp_attn_core_bwd_workspace(b, s, n_heads_local, d_head);
  if (!ws || ws_bytes < need)
    return fail(TP_ERR_WORKSPACE, "%s: workspace of %zu bytes required, got %zu%s", fn, need, ws_bytes,
                ws ? "" : " (NULL)");
  TRY(check_ptr(fn, "ws", ws));
  return hip_status(tps::attn_bwd(static_cast<const uint16_t*>(QKV), static_cast<const uint16_t*>(O),
                                  static_cast<const uint16_t*>(dO), lse, static_cast<uint16_t*>(dQKV), ws, (int)b,
                                  (int)s, (int)n_heads_local, (int)d_head,
                                  causal != 0, as_stream(stream)),
                    fn);
}

namespace {
// Stream-K area shared by the attention backward's four GEMMs.
size_t attn_bwd_sk(int64_t M, int64_t h, int64_t w) {
  return sk_max({sk_need(w, h, M), sk_need(M, w, h), sk_need(h, 3 * w, M), sk_need(M, h, 3 * w)});
}
}  // namespace

TP_API size_t tp_attn_bwd_workspace(int64_t b, int64_t s, int64_t h, int64_t n_heads_local, int64_t d_head) {
  if (b < 0 || s < 0 || n_heads_local < 0 || d_head < 0) return 0;
  const size_t t = (size_t)b * (size_t)s, w = (size_t)n_heads_local * (size_t)d_head;
  return round256(t * w * 2) + round256(t * 3 * w * 2) +
         round256(tp_attn_core_bwd_workspace(b, s, n_heads_local, d_head)) +
         attn_bwd_sk(b * s, h, n_heads_local * d_head);
}

TP_API tp_status tp_attn_bwd(int64_t b, int64_t s, int64_t h, int64_t n_heads_local, int64_t d_head, int causal,
                             const void* X, const void* Wqkv_i, const void* Wo_i, const void* QKV, const void* O,
                             const float* lse, const void* dOut, float* dX_i, float* dWqkv_i, float* dWo_i, void* ws,
                             size_t ws_bytes, void* stream) {
  const char* fn = "tp_attn_bwd";
  TRY(check_attn_shape(fn, b, s, n_heads_local, d_head));
  TRY(check_dims(fn, b * s, h, 3 * n_heads_local * d_head));
  TRY(check_ptr(fn, "dWqkv_i", dWqkv_i));
  TRY(check_ptr(fn, "dWo_i", dWo_i));
  const int64_t M = b * s, w = n_heads_local * d_head;
  if (M > 0) {
    TRY(check_ptr(fn, "X", X));
    TRY(check_ptr(fn, "Wqkv_i", Wqkv_i));
    TRY(check_ptr(fn, "Wo_i", Wo_i));
    TRY(check_ptr(fn, "QKV", QKV));
    TRY(check_ptr(fn, "O", O));
    TRY(check_ptr(fn, "lse", lse));
    TRY(check_ptr(fn, "dOut", dOut));
    TRY(check_ptr(fn, "dX_i", dX_i));
    TRY(check_attn_bytes(fn, M, h, w));
    TRY(check_bytes(fn, "dOut", M, h, 2));
  }
  const size_t need = tp_attn_bwd_workspace(b, s, h, n_heads_local, d_head);
  if (need && (!ws || ws_bytes < need))
    return fail(TP_ERR_WORKSPACE, "%s: workspace of %zu bytes required, got %zu%s", fn, need, ws_bytes,
                ws ? "" : " (NULL)");
  TRY(check_opt_ptr(fn, "ws", ws));
  hipStream_t st = as_stream(stream);
  char* wsb = static_cast<char*>(ws);
  uint16_t* dO = reinterpret_cast<uint16_t*>(wsb);
  uint16_t* dqkv = reinterpret_cast<uint16_t*>(wsb + round256((size_t)M * w * 2));
  void* core_ws = wsb + round256((size_t)M * w * 2) + round256((size_t)M * 3 * w * 2);
  void* sk = static_cast<char*>(core_ws) + round256(tp_attn_core_bwd_workspace(b, s, n_heads_local, d_head));
  {  // dWo_i = O^T dOut: A(m,k) = O[k, m], B(k,n) = dOut[k, n]
    tps::GemmArgs g = make_args(O, w, dOut, h, w, h, M, dWo_i, h);
    tps::gemm_bf16_sk_attach(g, sk);
    TRY(hip_status(tps::gemm_bf16(g, false, false, tps::EPI_F32, st), fn));
  }
  if (M > 0) {
    {  // dO = dOut Wo_i^T: A = dOut [M,h] (K-contig), B(k,n) = Wo_i[n, k] (K-contig)
      tps::GemmArgs g = make_args(dOut, h, Wo_i, h, M, w, h, dO, w);
      tps::gemm_bf16_sk_attach(g, sk);
      TRY(hip_status(tps::gemm_bf16(g, true, true, tps::EPI_BF16, st), fn));
    }
    TRY(hip_status(tps::attn_bwd(static_cast<const uint16_t*>(QKV), static_cast<const uint16_t*>(O), dO, lse, dqkv,
                                 core_ws, (int)b, (int)s, (int)n_heads_local, (int)d_head, causal != 0, st),
                   fn));
  }
  {  // dWqkv_i = X^T dQKV: A(m,k) = X[k, m], B(k,n) = dQKV[k, n]
    tps::GemmArgs g = make_args(X, h, dqkv, 3 * w, h, 3 * w, M, dWqkv_i, 3 * w);
    tps::gemm_bf16_sk_attach(g, sk);
    TRY(hip_status(tps::gemm_bf16(g, false, false, tps::EPI_F32, st), fn));
  }
  if (M > 0) {  // dX_i = dQKV Wqkv_i^T: A = dQKV [M,3w] (K-contig), B(k,n) = Wqkv_i[n, k] (K-contig)
    tps::GemmArgs g = make_args(dqkv, 3 * w, Wqkv_i, 3 * w, M, h, 3 * w, dX_i, h);
    tps::gemm_bf16_sk_attach(g, sk);
    TRY(hip_status(tps::gemm_bf16(g, true, true, tps::EPI_F32, st), fn));
  }
  return ok();
}

// float32 [M][ce_slots(V)][2]: (max, sum of exp) per row and column slot
static size_t ce_stats_bytes(int64_t M, int64_t V) { return (size_t)M * (size_t)tps::ce_slots((int)V) * 8; }

TP_API size_t tp_vocab_ce_workspace(int64_t M, int64_t h, int64_t lo, int64_t hi) {
  if (M < 0 || h <= 0 || lo < 0 || hi <= lo || hi - lo > kMaxDim) return 0;
  // the logits GEMM's per-slot row statistics, then its stream-K area (if it uses one)
  return round256(ce_stats_bytes(M, hi - lo)) + sk_need(M, hi - lo, h);
}

TP_API tp_status tp_vocab_ce_partials(int64_t M, int64_t h, int64_t lo, int64_t hi, const void* H, const void* E_i,
                                      const int32_t* targets, float* rowmax_i, float* sumexp_i, float* tlogit_i,
                                      void* ws, size_t ws_bytes, void* stream) {
  const char* fn = "tp_vocab_ce_partials";
  if (lo < 0 || lo >= hi)
    return fail(TP_ERR_INVALID_ARG, "%s: need 0 <= lo < hi (got lo=%lld hi=%lld)", fn, (long long)lo, (long long)hi);
  TRY(check_dims(fn, M, h, hi - lo));
  if (M == 0) return ok();
  TRY(check_ptr(fn, "H", H));
  TRY(check_ptr(fn, "E_i", E_i));
  if (!targets) return fail(TP_ERR_INVALID_ARG, "%s: targets is NULL", fn);
  TRY(check_ptr(fn, "rowmax_i", rowmax_i));
  TRY(check_ptr(fn, "sumexp_i", sumexp_i));
  TRY(check_ptr(fn, "tlogit_i", tlogit_i));
  TRY(check_bytes(fn, "H", M, h, 2));
  TRY(check_bytes(fn, "E_i", hi - lo, h, 2));
  const size_t need = tp_vocab_ce_workspace(M, h, lo, hi);
  if (!ws || ws_bytes < need)
    return fail(TP_ERR_WORKSPACE, "%s: workspace of %zu bytes required, got %zu%s", fn, need, ws_bytes,
                ws ? "" : " (NULL)");
  TRY(check_ptr(fn, "ws", ws));
  hipStream_t st = as_stream(stream);
  const int64_t V = hi - lo;
  float* stats = static_cast<float*>(ws);
  // logits_i = H E_i^T (A = H [M,h] K-contig, B(k,n) = E_i[n, k] K-contig), reduced in
  // the GEMM's epilogue to per-slot row statistics; the logits are never stored.
  tps::GemmArgs g = make_args(H, h, E_i, h, M, V, h, stats, 0);
  g.ce_targets = targets;
  g.ce_lo = lo;
  g.ce_tlogit = tlogit_i;
  tps::gemm_bf16_sk_attach(g, static_cast<char*>(ws) + round256(ce_stats_bytes(M, V)));
  TRY(hip_status(tps::gemm_bf16(g, true, true, tps::EPI_CE, st), fn));
  return hip_status(
      tps::ce_merge(stats, M, tps::ce_slots((int)V), targets, lo, V, rowmax_i, sumexp_i, tlogit_i, st), fn);
}

TP_API tp_status tp_vocab_ce_loss(int64_t M, const float* const* rowmax_parts, const float* const* sumexp_parts,
                                  const float* const* tlogit_parts, int n_parts, float* loss_rows, float* loss_sum,
                                  void* stream) {
  const char* fn = "tp_vocab_ce_loss";
  if (M < 0) return fail(TP_ERR_INVALID_ARG, "%s: M < 0", fn);
  if (M > kMaxDim) return fail(TP_ERR_UNSUPPORTED, "%s: M exceeds 2^31-1", fn);
  if (n_parts < 1 || n_parts > tps::kCeMaxParts)
    return fail(TP_ERR_INVALID_ARG, "%s: n_parts must be in [1, %d] (got %d)", fn, tps::kCeMaxParts, n_parts);
  if (!rowmax_parts || !sumexp_parts || !tlogit_parts) return fail(TP_ERR_INVALID_ARG, "%s: part arrays are NULL", fn);
  TRY(check_ptr(fn, "loss_sum", loss_sum));
  tps::CeParts p{};
  if (M > 0) {
    TRY(check_ptr(fn, "loss_rows", loss_rows));
    for (int i = 0; i < n_parts; ++i) {
      TRY(check_ptr(fn, "rowmax_parts[i]", rowmax_parts[i]));
      TRY(check_ptr(fn, "sumexp_parts[i]", sumexp_parts[i]));
      TRY(check_ptr(fn, "tlogit_parts[i]", tlogit_parts[i]));
      p.m[i] = rowmax_parts[i];
      p.s[i] = sumexp_parts[i];
      p.t[i] = tlogit_parts[i];
    }
  }
  return hip_status(tps::ce_loss(p, n_parts, M, loss_rows, loss_sum, as_stream(stream)), fn);
}

TP_API tp_status tp_vocab_embed(const int32_t* ids, int64_t n_tokens, const void* E_i, int64_t lo, int64_t hi,
                                int64_t h, void* out, void* stream) {
  const char* fn = "tp_vocab_embed";
  if (n_tokens < 0) return fail(TP_ERR_INVALID_ARG, "%s: n_tokens < 0", fn);
  if (lo < 0 || lo >= hi) return fail(TP_ERR_INVALID_ARG, "%s: need 0 <= lo < hi (got lo=%lld hi=%lld)", fn,
                                      (long long)lo, (long long)hi);
  if (h <= 0) return fail(TP_ERR_INVALID_ARG, "%s: h must be > 0", fn);
  if (h % 8) return fail(TP_ERR_UNSUPPORTED, "%s: h must be a multiple of 8 (got %lld)", fn, (long long)h);
  if (n_tokens > kMaxDim) return fail(TP_ERR_UNSUPPORTED, "%s: n_tokens exceeds 2^31-1", fn);
  if (n_tokens == 0) return ok();
  if (!ids) return fail(TP_ERR_INVALID_ARG, "%s: ids is NULL", fn);
  TRY(check_ptr(fn, "E_i", E_i));
  TRY(check_ptr(fn, "out", out));
  return hip_status(tps::vocab_gather(ids, n_tokens, static_cast<const uint16_t*>(E_i), lo, hi, h,
                                      static_cast<uint16_t*>(out), as_stream(stream)),
                    fn);
}

// ---- sequence parallelism

static tp_status check_sp_h(const char* fn, int64_t h) {
  if (h <= 0) return fail(TP_ERR_INVALID_ARG, "%s: h must be > 0 (got %lld)", fn, (long long)h);
  if (h % 8) return fail(TP_ERR_UNSUPPORTED, "%s: h must be a multiple of 8 (got %lld)", fn, (long long)h);
  return TP_OK;
}

TP_API tp_status tp_layernorm(int64_t rows, int64_t h, const float* X, const float* gamma, const float* beta,
                              float eps, void* Y, void* stream) {
  const char* fn = "tp_layernorm";
  if (rows < 0) return fail(TP_ERR_INVALID_ARG, "%s: rows < 0", fn);
  TRY(check_sp_h(fn, h));
  if (h > tps::kLnMaxH)
    return fail(TP_ERR_UNSUPPORTED, "%s: h above %lld is not supported", fn, (long long)tps::kLnMaxH);
  if (!(eps >= 0.f)) return fail(TP_ERR_INVALID_ARG, "%s: eps must be >= 0", fn);
  if (rows > kMaxDim) return fail(TP_ERR_UNSUPPORTED, "%s: rows exceeds 2^31-1", fn);
  if (rows == 0) return ok();
  TRY(check_ptr(fn, "X", X));
  TRY(check_ptr(fn, "gamma", gamma));
  TRY(check_ptr(fn, "beta", beta));
  TRY(check_ptr(fn, "Y", Y));
  return hip_status(tps::layernorm_rows(X, rows, h, gamma, beta, eps, static_cast<uint16_t*>(Y), as_stream(stream)),
                    fn);
}

TP_API size_t tp_layernorm_bwd_workspace(int64_t rows, int64_t h) {
  if (rows < 0 || h <= 0) return 0;
  return tps::layernorm_bwd_workspace(rows, h);
}

TP_API tp_status tp_layernorm_bwd(int64_t rows, int64_t h, const float* X, const float* gamma, const float* dY,
                                  const float* dRes, float eps, float* dX, float* dgamma, float* dbeta, void* ws,
                                  size_t ws_bytes, void* stream) {
  const char* fn = "tp_layernorm_bwd";
  if (rows < 0) return fail(TP_ERR_INVALID_ARG, "%s: rows < 0", fn);
  TRY(check_sp_h(fn, h));
  if (h > tps::kLnBwdMaxH)
    return fail(TP_ERR_UNSUPPORTED, "%s: h above %lld is not supported", fn, (long long)tps::kLnBwdMaxH);
  if (!(eps >= 0.f)) return fail(TP_ERR_INVALID_ARG, "%s: eps must be >= 0", fn);
  if (rows > kMaxDim) return fail(TP_ERR_UNSUPPORTED, "%s: rows exceeds 2^31-1", fn);
  TRY(check_ptr(fn, "gamma", gamma));
  TRY(check_ptr(fn, "dgamma", dgamma));
  TRY(check_ptr(fn, "dbeta", dbeta));
  if (rows > 0) {
    TRY(check_ptr(fn, "X", X));
    TRY(check_ptr(fn, "dY", dY));
    TRY(check_opt_ptr(fn, "dRes", dRes));
    TRY(check_ptr(fn, "dX", dX));
  }
  const size_t need = tp_layernorm_bwd_workspace(rows, h);
  if (!ws || ws_bytes < need)
    return fail(TP_ERR_WORKSPACE, "%s: workspace of %zu bytes required, got %zu%s", fn, need, ws_bytes,
                ws ? "" : " (NULL)");
  TRY(check_ptr(fn, "ws", ws));
  return hip_status(tps::layernorm_bwd(X, rows, h, gamma, dY, dRes, eps, dX, dgamma, dbeta, ws, as_stream(stream)),
                    fn);
}

TP_API tp_status tp_sp_dropout_bwd(int64_t rows, int64_t h, const float* dY, const uint8_t* keep, float keep_prob,
                                   void* out, void* stream) {
  const char* fn = "tp_sp_dropout_bwd";
  if (rows < 0) return fail(TP_ERR_INVALID_ARG, "%s: rows < 0", fn);
  TRY(check_sp_h(fn, h));
  if (keep && !(keep_prob > 0.f && keep_prob <= 1.f))
    return fail(TP_ERR_INVALID_ARG, "%s: keep_prob must be in (0, 1]", fn);
  if (keep && (reinterpret_cast<uintptr_t>(keep) & 3u))
    return fail(TP_ERR_UNSUPPORTED, "%s: keep is not 4-byte aligned", fn);
  if (rows == 0) return ok();
  TRY(check_ptr(fn, "dY", dY));
  TRY(check_ptr(fn, "out", out));
  return hip_status(tps::sp_dropout_bwd(dY, rows, h, keep, keep_prob, static_cast<uint16_t*>(out), as_stream(stream)),
                    fn);
}

TP_API tp_status tp_sp_reduce_scatter(int n_parts, const float* const* partials, int64_t s, int64_t h, int rank,
                                      const float* residual, const uint8_t* keep, float keep_prob, float* out,
                                      void* stream) {
  const char* fn = "tp_sp_reduce_scatter";
  if (n_parts < 1 || n_parts > tps::kSpMaxParts)
    return fail(TP_ERR_INVALID_ARG, "%s: n_parts must be in [1, %d] (got %d)", fn, tps::kSpMaxParts, n_parts);
  if (s < 0 || s % n_parts)
    return fail(TP_ERR_INVALID_ARG, "%s: s must be >= 0 and a multiple of n_parts (got s=%lld)", fn, (long long)s);
  TRY(check_sp_h(fn, h));
  if (rank < 0 || rank >= n_parts) return fail(TP_ERR_INVALID_ARG, "%s: rank %d outside [0, %d)", fn, rank, n_parts);
  if (keep && !(keep_prob > 0.f && keep_prob <= 1.f))
    return fail(TP_ERR_INVALID_ARG, "%s: keep_prob must be in (0, 1]", fn);
  if (keep && (reinterpret_cast<uintptr_t>(keep) & 3u))
    return fail(TP_ERR_UNSUPPORTED, "%s: keep is not 4-byte aligned", fn);
  const int64_t rows = s / n_parts;
  if (rows * h == 0) return ok();
  if (!partials) return fail(TP_ERR_INVALID_ARG, "%s: partials is NULL", fn);
  tps::SpParts p{};
  for (int i = 0; i < n_parts; ++i) {
    char name[32];
    snprintf(name, sizeof name, "partials[%d]", i);
    TRY(check_ptr(fn, name, partials[i]));
    p.p[i] = partials[i];
  }
  TRY(check_opt_ptr(fn, "residual", residual));
  TRY(check_ptr(fn, "out", out));
  return hip_status(tps::sp_reduce_scatter(p, n_parts, (int64_t)rank * rows, rows, h, residual, keep, keep_prob, out,
                                           as_stream(stream)),
                    fn);
}

TP_API tp_status tp_sp_all_gather(int n_parts, const void* const* slices, int64_t rows, int64_t h, void* out,
                                  void* stream) {
  const char* fn = "tp_sp_all_gather";
  if (n_parts < 1 || n_parts > tps::kSpMaxParts)
    return fail(TP_ERR_INVALID_ARG, "%s: n_parts must be in [1, %d] (got %d)", fn, tps::kSpMaxParts, n_parts);
  if (rows < 0) return fail(TP_ERR_INVALID_ARG, "%s: rows < 0", fn);
  TRY(check_sp_h(fn, h));
  if (rows == 0) return ok();
  if (!slices) return fail(TP_ERR_INVALID_ARG, "%s: slices is NULL", fn);
  tps::SpParts p{};
  for (int i = 0; i < n_parts; ++i) {
    char name[32];
    snprintf(name, sizeof name, "slices[%d]", i);
    TRY(check_ptr(fn, name, slices[i]));
    p.p[i] = slices[i];
  }
  TRY(check_ptr(fn, "out", out));
  return hip_status(tps::sp_all_gather(p, n_parts, rows, h, static_cast<uint16_t*>(out), as_stream(stream)), fn);
}

TP_API tp_status tp_shard_sum(tp_dtype dt, const void* const* partials, int n_partials, int64_t numel, void* out,
                              void* stream) {
  const char* fn = "tp_shard_sum";
  if (dt != TP_F32 && dt != TP_BF16) return fail(TP_ERR_INVALID_ARG, "%s: unknown dtype %d", fn, (int)dt);
  if (n_partials < 1 || n_partials > tps::kMaxPartials)
    return fail(TP_ERR_INVALID_ARG, "%s: n_partials must be in [1, %d] (got %d)", fn, tps::kMaxPartials, n_partials);
  if (numel < 0) return fail(TP_ERR_INVALID_ARG, "%s: numel < 0", fn);
  if (numel == 0) return ok();
  if (!partials) return fail(TP_ERR_INVALID_ARG, "%s: partials is NULL", fn);
  tps::SumArgs a{};
  for (int i = 0; i < n_partials; ++i) {
    char name[32];
    snprintf(name, sizeof name, "partials[%d]", i);
    TRY(check_ptr(fn, name, partials[i]));
    a.p[i] = partials[i];
  }
  TRY(check_ptr(fn, "out", out));
  a.n = n_partials;
  a.numel = numel;
  a.out = out;
  return hip_status(tps::shard_sum(a, dt == TP_BF16, as_stream(stream)), fn);
}
