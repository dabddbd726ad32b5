// Host-side interface of the vocabulary-parallel cross-entropy kernels (internal to libtpshard).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tps {
// Merge of the per-slot row statistics that the logits GEMM's EPI_CE epilogue
// leaves in part, float32 [M][nslot][2] (slot maximum, sum of exp relative to
// it): rowmax[m] = max over slots, sumexp[m] = sum_k s_k exp(m_k - rowmax[m]);
// tlogit[m] = 0 for the rows whose target lies outside [lo, lo + V) (the epilogue
// has stored the others).
hipError_t ce_merge(const float* part, int64_t M, int nslot, const int32_t* targets, int64_t lo, int64_t V,
                    float* rowmax, float* sumexp, float* tlogit, hipStream_t st);

constexpr int kCeMaxParts = 16;
struct CeParts {
  const float* m[kCeMaxParts];
  const float* s[kCeMaxParts];
  const float* t[kCeMaxParts];
};
// mx = max_i rowmax_i, S = sum_i sumexp_i exp(rowmax_i - mx) (order 0..n-1),
// loss_rows[m] = mx + log S[m] - sum_i tlogit_i[m],
// loss_sum = sum_m loss_rows[m] (one workgroup, fixed reduction tree).
hipError_t ce_loss(const CeParts& parts, int n, int64_t M, float* loss_rows, float* loss_sum, hipStream_t st);
}  // namespace tps
