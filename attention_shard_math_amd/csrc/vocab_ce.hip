// Vocabulary-parallel cross-entropy on top of the logits GEMM (gfx950).
//
// Rank i holds the logits of its vocabulary slice [lo, lo+V). Per token row it
// needs only the sum of exp over its own columns and, if it holds the row's
// target, that target's logit; the rows' softmax denominators are the sums of
// those partial sums over the ranks, and each row's loss is log(sum) - logit_t.
// The sums are carried relative to a row maximum so that no logit overflows
// float32: rank i keeps m_i = max of its columns and s_i = sum exp(logit - m_i),
// and the combine forms sum_i s_i exp(m_i - m) with m = max_i m_i (the max is
// one more all-reduce); in real arithmetic that equals the plain sum of exp.
//
// ce_rows: one wave per row, 16-byte loads strided over the lanes (each load
// instruction reads 1 KiB of the row, four in flight per lane); each lane keeps
// a running (max, rescaled sum) in float32, and the lanes' pairs are merged in a
// fixed butterfly. It is HBM-bound: 4*V bytes read per row.
// ce_loss: one workgroup; the partials are merged in rank order and the row
// losses reduced through LDS in a fixed tree, so the scalar is reproducible.
#include "common.hpp"
#include "vocab_ce.hpp"

namespace tps {
namespace {

// Running (max, sum of exp relative to it) of a lane: absorb values whose
// maximum is mx.
__device__ __forceinline__ void absorb_max(float& m, float& acc, float mx) {
  if (mx > m) {
    acc = (m == -__builtin_huge_valf()) ? 0.f : acc * expf(m - mx);
    m = mx;
  }
}

__global__ __launch_bounds__(256) void ce_rows_kernel(const float* __restrict__ logits, int64_t M, int V,
                                                      const int32_t* __restrict__ targets, int64_t lo,
                                                      float* __restrict__ rowmax, float* __restrict__ sumexp,
                                                      float* __restrict__ tlogit) {
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= M) return;  // whole wave
  const float* r = logits + row * (int64_t)V;
  float m = -__builtin_huge_valf(), acc = 0.f;
  if ((V & 3) == 0) {  // rows start 16-byte aligned
    const f32x4* r4 = reinterpret_cast<const f32x4*>(r);
    const int n4 = V >> 2;
    int i = lane;
    // Four loads in flight per lane (one wave per row leaves few waves per SIMD
    // to hide the latency).
    for (; i + 192 < n4; i += 256) {
      f32x4 x[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) x[u] = r4[i + 64 * u];
      float mx = m;
#pragma unroll
      for (int u = 0; u < 4; ++u) mx = fmaxf(mx, fmaxf(fmaxf(x[u][0], x[u][1]), fmaxf(x[u][2], x[u][3])));
      absorb_max(m, acc, mx);
#pragma unroll
      for (int u = 0; u < 4; ++u)
        acc += (expf(x[u][0] - m) + expf(x[u][1] - m)) + (expf(x[u][2] - m) + expf(x[u][3] - m));
    }
    for (; i < n4; i += 64) {
      const f32x4 x = r4[i];
      absorb_max(m, acc, fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])));
      acc += (expf(x[0] - m) + expf(x[1] - m)) + (expf(x[2] - m) + expf(x[3] - m));
    }
  } else {
    for (int i = lane; i < V; i += 64) {
      absorb_max(m, acc, r[i]);
      acc += expf(r[i] - m);
    }
  }
  // merge the lanes' pairs in a fixed butterfly (lanes without values carry -inf, 0)
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float mo = __shfl_xor(m, o), ao = __shfl_xor(acc, o);
    const float mn = fmaxf(m, mo);
    if (mn != -__builtin_huge_valf()) acc = acc * expf(m - mn) + ao * expf(mo - mn);
    m = mn;
  }
  if (lane == 0) {
    rowmax[row] = m;
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
    float mx = p.m[0][m];
    for (int i = 1; i < n; ++i) mx = fmaxf(mx, p.m[i][m]);
    float S = 0.f, T = 0.f;
    for (int i = 0; i < n; ++i) {
      S += p.s[i][m] * expf(p.m[i][m] - mx);
      T += p.t[i][m];
    }
    const float l = (mx + logf(S)) - T;
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

hipError_t ce_rows(const float* logits, int64_t M, int V, const int32_t* targets, int64_t lo, float* rowmax,
                   float* sumexp, float* tlogit, hipStream_t st) {
  if (M <= 0) return hipSuccess;
  const int64_t blocks = (M + 3) / 4;
  hipLaunchKernelGGL(ce_rows_kernel, dim3((unsigned)blocks), dim3(256), 0, st, logits, M, V, targets, lo, rowmax,
                     sumexp, tlogit);
  return hipGetLastError();
}

hipError_t ce_loss(const CeParts& parts, int n, int64_t M, float* loss_rows, float* loss_sum, hipStream_t st) {
  hipLaunchKernelGGL(ce_loss_kernel, dim3(1), dim3(1024), 0, st, parts, n, M, loss_rows, loss_sum);
  return hipGetLastError();
}

}  // namespace tps
