// Vocabulary-parallel cross-entropy on top of the logits GEMM (gfx950).
//
// Rank i holds the logits of its vocabulary slice [lo, lo+V). Per token row it
// needs only the sum of exp over its own columns and, if it holds the row's
// target, that target's logit; the rows' softmax denominators are the sums of
// those partial sums over the ranks, and each row's loss is log(sum) - logit_t.
//
// ce_rows: one wave per row, 16-byte loads strided over the lanes (each load
// instruction reads 1 KiB of the row, four in flight per lane), exp in float32,
// the lanes' partial sums added in a fixed butterfly. It is HBM-bound: 4*V
// bytes read per row.
// ce_loss: one workgroup; the partial sums are added in rank order and the
// row losses reduced through LDS in a fixed tree, so the scalar is reproducible.
#include "common.hpp"
#include "vocab_ce.hpp"

namespace tps {
namespace {

__global__ __launch_bounds__(256) void ce_rows_kernel(const float* __restrict__ logits, int64_t M, int V,
                                                      const int32_t* __restrict__ targets, int64_t lo,
                                                      float* __restrict__ sumexp, float* __restrict__ tlogit) {
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= M) return;  // whole wave
  const float* r = logits + row * (int64_t)V;
  float acc = 0.f;
  if ((V & 3) == 0) {  // rows start 16-byte aligned
    const f32x4* r4 = reinterpret_cast<const f32x4*>(r);
    const int n4 = V >> 2;
    int i = lane;
    // Four loads in flight per lane (one wave per row leaves few waves per SIMD
    // to hide the latency); the additions keep the order of the plain loop.
    for (; i + 192 < n4; i += 256) {
      f32x4 x[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) x[u] = r4[i + 64 * u];
#pragma unroll
      for (int u = 0; u < 4; ++u) acc += (expf(x[u][0]) + expf(x[u][1])) + (expf(x[u][2]) + expf(x[u][3]));
    }
    for (; i < n4; i += 64) {
      const f32x4 x = r4[i];
      acc += (expf(x[0]) + expf(x[1])) + (expf(x[2]) + expf(x[3]));
    }
  } else {
    for (int i = lane; i < V; i += 64) acc += expf(r[i]);
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) acc += __shfl_xor(acc, o);
  if (lane == 0) {
    sumexp[row] = acc;
    const int64_t t = targets[row];
    tlogit[row] = (t >= lo && t < lo + V) ? r[t - lo] : 0.f;
  }
}

__global__ __launch_bounds__(1024) void ce_loss_kernel(CeParts p, int n, int64_t M, float* __restrict__ loss_rows,
                                                       float* __restrict__ loss_sum) {
  __shared__ float red[1024];
  float part = 0.f;
  for (int64_t m = threadIdx.x; m < M; m += 1024) {
    float S = 0.f, T = 0.f;
    for (int i = 0; i < n; ++i) {
      S += p.s[i][m];
      T += p.t[i][m];
    }
    const float l = logf(S) - T;
    loss_rows[m] = l;
    part += l;
  }
  red[threadIdx.x] = part;
  __syncthreads();
  for (int w = 512; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) *loss_sum = red[0];
}

}  // namespace

hipError_t ce_rows(const float* logits, int64_t M, int V, const int32_t* targets, int64_t lo, float* sumexp,
                   float* tlogit, hipStream_t st) {
  if (M <= 0) return hipSuccess;
  const int64_t blocks = (M + 3) / 4;
  hipLaunchKernelGGL(ce_rows_kernel, dim3((unsigned)blocks), dim3(256), 0, st, logits, M, V, targets, lo, sumexp,
                     tlogit);
  return hipGetLastError();
}

hipError_t ce_loss(const CeParts& parts, int n, int64_t M, float* loss_rows, float* loss_sum, hipStream_t st) {
  hipLaunchKernelGGL(ce_loss_kernel, dim3(1), dim3(1024), 0, st, parts, n, M, loss_rows, loss_sum);
  return hipGetLastError();
}

}  // namespace tps
