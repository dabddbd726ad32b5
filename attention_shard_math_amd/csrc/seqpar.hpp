// Host-side interface of the sequence-parallel kernels (internal to libtpshard).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tps {

constexpr int kSpMaxParts = 16;
constexpr int kLnThreads = 1024;    // threads of a LayerNorm row workgroup
constexpr int64_t kLnMaxH = 32768;  // 8 float4 per thread of a row

// Y[r] = bf16((X[r] - mean) / sqrt(var + eps) * gamma + beta), one row per workgroup.
// X float32 [rows, h], gamma/beta float32 [h], h % 4 == 0, h <= kLnMaxH.
hipError_t layernorm_rows(const float* X, int64_t rows, int64_t h, const float* gamma, const float* beta, float eps,
                          uint16_t* Y, hipStream_t st);

constexpr int64_t kLnBwdMaxH = 24576;  // 6 float4 per thread for each of X and dY
constexpr int kLnBwdRowBlocks = 64;    // row blocks of the gamma/beta column sums

// Backward of layernorm_rows over rows x h (float32 X, dY): dX (+ dRes if not null),
// dgamma and dbeta [h] (overwritten). ws: layernorm_bwd_workspace(rows, h) bytes.
size_t layernorm_bwd_workspace(int64_t rows, int64_t h);
hipError_t layernorm_bwd(const float* X, int64_t rows, int64_t h, const float* gamma, const float* dY,
                         const float* dRes, float eps, float* dX, float* dgamma, float* dbeta, void* ws,
                         hipStream_t st);

// out (bf16) = keep ? dY / keep_prob : 0 (keep == nullptr: out = dY), rows x h float32 dY.
hipError_t sp_dropout_bwd(const float* dY, int64_t rows, int64_t h, const uint8_t* keep, float keep_prob,
                          uint16_t* out, hipStream_t st);

struct SpParts {
  const void* p[kSpMaxParts];
};

// out[r, :] = residual[r, :] + dropout(sum_j P_j[row0 + r, :]) over rows x h (h % 4 == 0);
// residual == nullptr: no residual add.
// keep == nullptr: no dropout. Otherwise kept values are divided by keep_prob.
hipError_t sp_reduce_scatter(const SpParts& parts, int n, int64_t row0, int64_t rows, int64_t h,
                             const float* residual, const uint8_t* keep, float keep_prob, float* out, hipStream_t st);

// out = [S_0; S_1; ...; S_{n-1}], each S_j bf16 [rows, h] (rows*h % 8 == 0).
hipError_t sp_all_gather(const SpParts& parts, int n, int64_t rows, int64_t h, uint16_t* out, hipStream_t st);

}  // namespace tps
