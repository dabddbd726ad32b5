// HBM-bound kernels of the rank-shard path:
//  * shard_sum — the all-reduce stand-in: out = ((P_0 + P_1) + ...) + P_{N-1}
//    elementwise in float32, fixed order, for float32 or bf16 partials;
//  * vocab_gather — the vocabulary-parallel input embedding: copy row
//    ids[t] - lo of the rank's table slice, or write a zero row when the id is
//    outside [lo, hi).
// Both stream 16-byte vectors with non-temporal accesses (each byte is touched
// once) and use a grid sized to keep every CU busy with several waves.
#include "bandwidth.hpp"
#include "common.hpp"

namespace tps {
namespace {

// Each thread sums U vectors (256 apart) per partial per iteration, so every
// thread has N*U 16-byte loads in flight (the kernel is HBM-bound); U shrinks for
// large N to keep the loads within 128 VGPRs.
template <int N>
constexpr int sum_unroll() { return N <= 8 ? 4 : 2; }

template <int N>
__global__ __launch_bounds__(256) void shard_sum_f32_kernel(SumArgs a) {
  constexpr int kSumU = sum_unroll<N>();
  const int64_t nvec = a.numel >> 2;
  const int64_t stride = (int64_t)gridDim.x * 256 * kSumU;
  f32x4* out = static_cast<f32x4*>(a.out);
  for (int64_t v0 = (int64_t)blockIdx.x * 256 * kSumU + threadIdx.x; v0 < nvec; v0 += stride) {
    f32x4 x[kSumU][N];
#pragma unroll
    for (int u = 0; u < kSumU; ++u) {
      const int64_t v = v0 + u * 256;
#pragma unroll
      for (int i = 0; i < N; ++i)
        x[u][i] = v < nvec ? __builtin_nontemporal_load(static_cast<const f32x4*>(a.p[i]) + v) : f32x4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int u = 0; u < kSumU; ++u) {
      const int64_t v = v0 + u * 256;
      f32x4 s = x[u][0];
#pragma unroll
      for (int i = 1; i < N; ++i) s = s + x[u][i];
      if (v < nvec) __builtin_nontemporal_store(s, out + v);
    }
  }
  // tail (numel % 4 elements), one thread each
  const int64_t t = (nvec << 2) + (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t < a.numel && t < (nvec << 2) + 4) {
    float s = static_cast<const float*>(a.p[0])[t];
#pragma unroll
    for (int i = 1; i < N; ++i) s = s + static_cast<const float*>(a.p[i])[t];
    static_cast<float*>(a.out)[t] = s;
  }
}

template <int N>
__global__ __launch_bounds__(256) void shard_sum_bf16_kernel(SumArgs a) {
  const int64_t nvec = a.numel >> 3;  // 8 bf16 per 16-byte vector
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  u32x4* out = static_cast<u32x4*>(a.out);
  for (int64_t v = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; v < nvec; v += stride) {
    u32x4 x[N];
#pragma unroll
    for (int i = 0; i < N; ++i) x[i] = __builtin_nontemporal_load(static_cast<const u32x4*>(a.p[i]) + v);
    u32x4 r;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      float lo = bf16_bits_to_f32(x[0][w] & 0xffffu), hi = bf16_bits_to_f32(x[0][w] >> 16);
#pragma unroll
      for (int i = 1; i < N; ++i) {
        lo = lo + bf16_bits_to_f32(x[i][w] & 0xffffu);
        hi = hi + bf16_bits_to_f32(x[i][w] >> 16);
      }
      r[w] = pack_bf16x2(lo, hi);
    }
    __builtin_nontemporal_store(r, out + v);
  }
  const int64_t t = (nvec << 3) + (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t < a.numel && t < (nvec << 3) + 8) {
    float s = bf16_bits_to_f32(static_cast<const uint16_t*>(a.p[0])[t]);
#pragma unroll
    for (int i = 1; i < N; ++i) s = s + bf16_bits_to_f32(static_cast<const uint16_t*>(a.p[i])[t]);
    static_cast<uint16_t*>(a.out)[t] = (uint16_t)f32_to_bf16_bits(s);
  }
}

template <int N>
hipError_t launch_sum(const SumArgs& a, bool bf16, hipStream_t s) {
  const int64_t per = bf16 ? 8 : 4;
  const int64_t nvec = a.numel / per;
  const int64_t chunk = bf16 ? 256 : 256 * sum_unroll<N>();  // vectors per workgroup per iteration
  int64_t blocks = (nvec + chunk - 1) / chunk;
  const int64_t cap = bf16 ? 256 * 16 : 256 * 8;  // enough workgroups to keep every CU busy
  if (blocks > cap) blocks = cap;
  if (blocks < 1) blocks = 1;
  if (bf16)
    hipLaunchKernelGGL(shard_sum_bf16_kernel<N>, dim3((unsigned)blocks), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(shard_sum_f32_kernel<N>, dim3((unsigned)blocks), dim3(256), 0, s, a);
  return hipGetLastError();
}

// One workgroup per token row: h/8 16-byte vectors, strided over 256 threads.
__global__ __launch_bounds__(256) void vocab_gather_kernel(const int32_t* __restrict__ ids, const u32x4* __restrict__ E,
                                                           int64_t lo, int64_t hi, int64_t hvec,
                                                           u32x4* __restrict__ out) {
  const int64_t t = blockIdx.x;
  const int64_t id = ids[t];
  u32x4* o = out + t * hvec;
  if (id >= lo && id < hi) {
    const u32x4* src = E + (id - lo) * hvec;
    for (int64_t v = threadIdx.x; v < hvec; v += 256) __builtin_nontemporal_store(src[v], o + v);
  } else {
    const u32x4 z = {0u, 0u, 0u, 0u};
    for (int64_t v = threadIdx.x; v < hvec; v += 256) __builtin_nontemporal_store(z, o + v);
  }
}

}  // namespace

hipError_t shard_sum(const SumArgs& a, bool bf16, hipStream_t s) {
  if (a.numel == 0) return hipSuccess;
  switch (a.n) {
#define TPS_CASE(k) \
  case k:           \
    return launch_sum<k>(a, bf16, s);
    TPS_CASE(1) TPS_CASE(2) TPS_CASE(3) TPS_CASE(4) TPS_CASE(5) TPS_CASE(6) TPS_CASE(7) TPS_CASE(8)
    TPS_CASE(9) TPS_CASE(10) TPS_CASE(11) TPS_CASE(12) TPS_CASE(13) TPS_CASE(14) TPS_CASE(15) TPS_CASE(16)
#undef TPS_CASE
    default:
      return hipErrorInvalidValue;
  }
}

hipError_t vocab_gather(const int32_t* ids, int64_t n_tokens, const uint16_t* E, int64_t lo, int64_t hi, int64_t h,
                        uint16_t* out, hipStream_t s) {
  if (n_tokens == 0) return hipSuccess;
  hipLaunchKernelGGL(vocab_gather_kernel, dim3((unsigned)n_tokens), dim3(256), 0, s, ids,
                     reinterpret_cast<const u32x4*>(E), lo, hi, h / 8, reinterpret_cast<u32x4*>(out));
  return hipGetLastError();
}

}  // namespace tps
