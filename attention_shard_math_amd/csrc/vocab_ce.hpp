// Host-side interface of the vocabulary-parallel cross-entropy kernels (internal to libtpshard).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tps {
// Per row m of logits [M, V] (float32, row-major): rowmax[m] = max_n logits[m, n],
// sumexp[m] = sum_n exp(logits[m, n] - rowmax[m]); tlogit[m] = logits[m, t - lo] when
// lo <= t = targets[m] < lo + V, else 0.
hipError_t ce_rows(const float* logits, int64_t M, int V, const int32_t* targets, int64_t lo, float* rowmax,
                   float* sumexp, float* tlogit, hipStream_t st);

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
