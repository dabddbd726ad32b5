// Host-side interface of the shard-sum and vocab-gather kernels (internal).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tps {

constexpr int kMaxPartials = 16;

struct SumArgs {
  const void* p[kMaxPartials];
  int n;
  int64_t numel;
  void* out;
};

// out = ((p0 + p1) + ...) + p_{n-1} in float32 (bf16: widened, summed, rounded once).
hipError_t shard_sum(const SumArgs& a, bool bf16, hipStream_t s);

// out[t] = E[ids[t] - lo] if lo <= ids[t] < hi else 0; rows of h bf16 (h % 8 == 0).
hipError_t vocab_gather(const int32_t* ids, int64_t n_tokens, const uint16_t* E, int64_t lo, int64_t hi, int64_t h,
                        uint16_t* out, hipStream_t s);

}  // namespace tps
