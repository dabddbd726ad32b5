// Host-side interface of the sequence-parallel kernels (internal to libtpshard).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tps {

constexpr int kSpMaxParts = 16;
constexpr int64_t kLnMaxH = 32768;  // 32 float4 per thread of a 256-thread row

// Y[r] = bf16((X[r] - mean) / sqrt(var + eps) * gamma + beta), one row per workgroup.
// X float32 [rows, h], gamma/beta float32 [h], h % 4 == 0, h <= kLnMaxH.
hipError_t layernorm_rows(const float* X, int64_t rows, int64_t h, const float* gamma, const float* beta, float eps,
                          uint16_t* Y, hipStream_t st);

struct SpParts {
  const void* p[kSpMaxParts];
};

// out[r, :] = residual[r, :] + dropout(sum_j P_j[row0 + r, :]) over rows x h (h % 4 == 0).
// keep == nullptr: no dropout. Otherwise kept values are divided by keep_prob.
hipError_t sp_reduce_scatter(const SpParts& parts, int n, int64_t row0, int64_t rows, int64_t h,
                             const float* residual, const uint8_t* keep, float keep_prob, float* out, hipStream_t st);

// out = [S_0; S_1; ...; S_{n-1}], each S_j bf16 [rows, h] (rows*h % 8 == 0).
hipError_t sp_all_gather(const SpParts& parts, int n, int64_t rows, int64_t h, uint16_t* out, hipStream_t st);

}  // namespace tps
