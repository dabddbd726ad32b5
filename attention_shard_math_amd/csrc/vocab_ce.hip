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
// The logits themselves are never stored: the logits GEMM's epilogue reduces each
// row over each 48-column slot (half of a wave's 96-column block) to (slot max, sum
// of exp relative to it) and stores the target logits of the rows whose target
// lies in the slice; ce_merge combines a row's slots in a fixed order (one wave
// per row) and zeroes the target logit of the other rows. ce_loss: one workgroup; the partials are merged
// in rank order and the row losses reduced through LDS in a fixed tree, so the
// scalar is reproducible.
#include "common.hpp"
#include "gemm_bf16.hpp"
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

// One wave per row; lane k merges slots k, k + 64, ... then the lanes' pairs are
// merged in a fixed butterfly (lanes without values carry -inf, 0).
__global__ __launch_bounds__(256) void ce_merge_kernel(const f32x2* __restrict__ part, int64_t M, int nslot,
                                                       const int32_t* __restrict__ targets, int64_t lo, int64_t V,
                                                       float* __restrict__ rowmax, float* __restrict__ sumexp,
                                                       float* __restrict__ tlogit) {
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= M) return;  // whole wave
  const f32x2* r = part + row * (int64_t)nslot;
  float m = -__builtin_huge_valf(), acc = 0.f;
  for (int k = lane; k < nslot; k += 64) {
    const f32x2 x = r[k];
    if (x[0] == -__builtin_huge_valf()) continue;  // a slot wholly past the slice's end
    absorb_max(m, acc, x[0]);
    acc += x[1] * expf(x[0] - m);
  }
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
    const int64_t t = (int64_t)targets[row] - lo;
    if (t < 0 || t >= V) tlogit[row] = 0.f;  // in the slice: stored by the GEMM's epilogue
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

hipError_t ce_merge(const float* part, int64_t M, int nslot, const int32_t* targets, int64_t lo, int64_t V,
                    float* rowmax, float* sumexp, float* tlogit, hipStream_t st) {
  if (M <= 0) return hipSuccess;
  const int64_t blocks = (M + 3) / 4;
  hipLaunchKernelGGL(ce_merge_kernel, dim3((unsigned)blocks), dim3(256), 0, st, reinterpret_cast<const f32x2*>(part),
                     M, nslot, targets, lo, V, rowmax, sumexp, tlogit);
  return hipGetLastError();
}

hipError_t ce_loss(const CeParts& parts, int n, int64_t M, float* loss_rows, float* loss_sum, hipStream_t st) {
  hipLaunchKernelGGL(ce_loss_kernel, dim3(1), dim3(1024), 0, st, parts, n, M, loss_rows, loss_sum);
  return hipGetLastError();
}

}  // namespace tps
