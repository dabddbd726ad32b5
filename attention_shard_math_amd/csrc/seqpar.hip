// Sequence-parallel kernels around the tensor-parallel MLP (gfx950).
//
// With sequence parallelism the light row-wise operators run on one rank's
// contiguous slice of the sequence, and the MLP's all-reduce is split into its
// two halves: an all-gather of the LayerNorm output before the column GEMM and
// a reduce-scatter of the fp32 partials after the row GEMM. On one GPU the two
// collectives are stand-ins that move the same bytes:
//  * layernorm_rows — one 1024-thread workgroup per row (16 waves, so that a
//    CU has four times the loads of a 256-thread row in flight from the start).
//    The row stays in registers (up to 8 float4 per thread), so HBM sees one
//    read of X and one bf16 write of Y; mean, then the biased variance from the
//    held values (two-pass, no cancellation), each reduced with a fixed
//    butterfly per wave and a fixed order over the waves.
//  * sp_reduce_scatter — rank-ordered float32 sum of the N partials over the
//    rank's rows, dropout with an input keep mask, residual add; 16-byte
//    non-temporal accesses. HBM-bound: (4N + 4 + 1 + 4) bytes per element.
//  * sp_all_gather — N slice copies into the gathered buffer in one launch.
// Backward:
//  * layernorm_bwd_rows — one workgroup per row, X and dY rows in registers:
//    dX = rstd (g - mean(g) - xh mean(g xh)) (+ the residual path's gradient),
//    g = dY gamma, xh = (x - mean) rstd; the row's mean and rstd are kept for
//    the column sums;
//  * layernorm_bwd_cols — dgamma = sum_rows dY xh, dbeta = sum_rows dY, as
//    partial sums over 64 row blocks (fixed order), then colsum: 16 threads per
//    column each add a sixteenth of the blocks in order, and the 16 part sums
//    are added in part order (a fixed order, so repeated calls agree bit for bit);
//  * dropout_bwd — dY / p where kept, else 0, rounded to bf16 (the MLP
//    backward's input); the all-gather and reduce-scatter above serve the
//    backward unchanged (each is the other's backward).
#include <type_traits>

#include "common.hpp"
#include "seqpar.hpp"

namespace tps {
namespace {

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// Sum over the NT threads of the workgroup: butterfly per wave, then the wave
// sums added in wave order by every thread.
template <int NT>
__device__ __forceinline__ float block_sum(float v, float* red) {
  v = wave_sum(v);
  __syncthreads();  // red may still be read from the previous call
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  float s = red[0];
#pragma unroll
  for (int w = 1; w < NT / 64; ++w) s += red[w];
  return s;
}

template <int VPT, int NT>
__global__ __launch_bounds__(NT) void layernorm_kernel(const f32x4* __restrict__ X, int64_t h4,
                                                       const f32x4* __restrict__ gamma,
                                                       const f32x4* __restrict__ beta, float eps, float inv_h,
                                                       uint2* __restrict__ Y) {
  __shared__ float red[NT / 64];
  const int64_t row = blockIdx.x;
  const f32x4* x = X + row * h4;
  f32x4 v[VPT];
  float s = 0.f;
#pragma unroll
  for (int k = 0; k < VPT; ++k) {
    const int64_t j = threadIdx.x + k * NT;
    v[k] = j < h4 ? __builtin_nontemporal_load(x + j) : f32x4{0.f, 0.f, 0.f, 0.f};
    s += (v[k][0] + v[k][1]) + (v[k][2] + v[k][3]);
  }
  const float mean = block_sum<NT>(s, red) * inv_h;
  float q = 0.f;
#pragma unroll
  for (int k = 0; k < VPT; ++k) {
    const int64_t j = threadIdx.x + k * NT;
    if (j < h4) {
      const float d0 = v[k][0] - mean, d1 = v[k][1] - mean, d2 = v[k][2] - mean, d3 = v[k][3] - mean;
      q += (d0 * d0 + d1 * d1) + (d2 * d2 + d3 * d3);
    }
  }
  const float var = block_sum<NT>(q, red) * inv_h;
  const float rstd = 1.0f / sqrtf(var + eps);
  uint2* y = Y + row * h4;
#pragma unroll
  for (int k = 0; k < VPT; ++k) {
    const int64_t j = threadIdx.x + k * NT;
    if (j < h4) {
      const f32x4 g = gamma[j], b = beta[j];
      const float y0 = (v[k][0] - mean) * rstd * g[0] + b[0];
      const float y1 = (v[k][1] - mean) * rstd * g[1] + b[1];
      const float y2 = (v[k][2] - mean) * rstd * g[2] + b[2];
      const float y3 = (v[k][3] - mean) * rstd * g[3] + b[3];
      y[j] = uint2{pack_bf16x2(y0, y1), pack_bf16x2(y2, y3)};
    }
  }
}

template <int VPT, int NT>
__global__ __launch_bounds__(NT) void layernorm_bwd_rows_kernel(const f32x4* __restrict__ X, int64_t h4,
                                                                const f32x4* __restrict__ gamma,
                                                                const f32x4* __restrict__ dY,
                                                                const f32x4* __restrict__ dRes, float eps,
                                                                float inv_h, f32x4* __restrict__ dX,
                                                                float2* __restrict__ stats) {
  __shared__ float red[NT / 64];
  const int64_t row = blockIdx.x;
  const f32x4* x = X + row * h4;
  const f32x4* dy = dY + row * h4;
  f32x4 v[VPT], gv[VPT];
  float sx = 0.f;
#pragma unroll
  for (int k = 0; k < VPT; ++k) {
    const int64_t j = threadIdx.x + k * NT;
    v[k] = j < h4 ? x[j] : f32x4{0.f, 0.f, 0.f, 0.f};
    gv[k] = j < h4 ? dy[j] * gamma[j] : f32x4{0.f, 0.f, 0.f, 0.f};
    sx += (v[k][0] + v[k][1]) + (v[k][2] + v[k][3]);
  }
  const float mean = block_sum<NT>(sx, red) * inv_h;
  float q = 0.f;
#pragma unroll
  for (int k = 0; k < VPT; ++k) {
    const int64_t j = threadIdx.x + k * NT;
    if (j < h4) {
      const float d0 = v[k][0] - mean, d1 = v[k][1] - mean, d2 = v[k][2] - mean, d3 = v[k][3] - mean;
      q += (d0 * d0 + d1 * d1) + (d2 * d2 + d3 * d3);
    }
  }
  const float rstd = 1.0f / sqrtf(block_sum<NT>(q, red) * inv_h + eps);
  float sg = 0.f, sgx = 0.f;
#pragma unroll
  for (int k = 0; k < VPT; ++k) {
    const int64_t j = threadIdx.x + k * NT;
    if (j < h4) {
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        v[k][c] = (v[k][c] - mean) * rstd;  // xh
        sg += gv[k][c];
        sgx += gv[k][c] * v[k][c];
      }
    }
  }
  const float mg = block_sum<NT>(sg, red) * inv_h;
  const float mgx = block_sum<NT>(sgx, red) * inv_h;
#pragma unroll
  for (int k = 0; k < VPT; ++k) {
    const int64_t j = threadIdx.x + k * NT;
    if (j < h4) {
      f32x4 o;
#pragma unroll
      for (int c = 0; c < 4; ++c) o[c] = rstd * (gv[k][c] - mg - v[k][c] * mgx);
      if (dRes) o = o + dRes[row * h4 + j];
      dX[row * h4 + j] = o;
    }
  }
  if (threadIdx.x == 0) stats[row] = float2{mean, rstd};
}

// Partial column sums over row block blockIdx.y (rows rb*rpb .. +rpb), in row order.
__global__ __launch_bounds__(256) void layernorm_bwd_cols_kernel(const f32x4* __restrict__ X,
                                                                 const f32x4* __restrict__ dY,
                                                                 const float2* __restrict__ stats, int64_t rows,
                                                                 int64_t h4, int64_t rpb, f32x4* __restrict__ pg,
                                                                 f32x4* __restrict__ pb) {
  const int64_t j = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (j >= h4) return;
  const int64_t r0 = (int64_t)blockIdx.y * rpb, r1 = min(rows, r0 + rpb);
  f32x4 ag = {0.f, 0.f, 0.f, 0.f}, ab = {0.f, 0.f, 0.f, 0.f};
  for (int64_t r = r0; r < r1; ++r) {
    const float2 st = stats[r];
    const f32x4 dy = dY[r * h4 + j], x = X[r * h4 + j];
#pragma unroll
    for (int c = 0; c < 4; ++c) ag[c] += dy[c] * ((x[c] - st.x) * st.y);
    ab = ab + dy;
  }
  pg[(int64_t)blockIdx.y * h4 + j] = ag;
  pb[(int64_t)blockIdx.y * h4 + j] = ab;
}

// Sum of the nb partial rows for 16 float4 columns per workgroup: the 16
// threads of a column take consecutive sixteenths of the blocks, each adding its
// blocks in order, and the 16 part sums are then added in part order.
__global__ __launch_bounds__(256) void colsum_kernel(const f32x4* __restrict__ pg, const f32x4* __restrict__ pb,
                                                     int nb, int64_t h4, f32x4* __restrict__ dgamma,
                                                     f32x4* __restrict__ dbeta) {
  __shared__ f32x4 sg[16][16], sb[16][16];
  const int c = threadIdx.x & 15, part = threadIdx.x >> 4;
  const int64_t j = (int64_t)blockIdx.x * 16 + c;
  f32x4 g = {0.f, 0.f, 0.f, 0.f}, b = {0.f, 0.f, 0.f, 0.f};
  if (j < h4) {
    const int i1 = (part + 1) * nb / 16;
#pragma unroll 4
    for (int i = part * nb / 16; i < i1; ++i) {
      g = g + pg[(int64_t)i * h4 + j];
      b = b + pb[(int64_t)i * h4 + j];
    }
  }
  sg[part][c] = g;
  sb[part][c] = b;
  __syncthreads();
  if (part == 0 && j < h4) {
#pragma unroll
    for (int q = 1; q < 16; ++q) {
      g = g + sg[q][c];
      b = b + sb[q][c];
    }
    dgamma[j] = g;
    dbeta[j] = b;
  }
}

__global__ __launch_bounds__(256) void dropout_bwd_kernel(const f32x4* __restrict__ dY,
                                                          const uint32_t* __restrict__ keep, float keep_prob,
                                                          int64_t nvec, uint2* __restrict__ out) {
  const int64_t stride = (int64_t)gridDim.x * 256;
  for (int64_t v = (int64_t)blockIdx.x * 256 + threadIdx.x; v < nvec; v += stride) {
    f32x4 g = dY[v];
    if (keep) {
      const uint32_t k = keep[v];
#pragma unroll
      for (int c = 0; c < 4; ++c) g[c] = ((k >> (8 * c)) & 0xffu) ? g[c] / keep_prob : 0.f;
    }
    out[v] = uint2{pack_bf16x2(g[0], g[1]), pack_bf16x2(g[2], g[3])};
  }
}

template <int N>
__global__ __launch_bounds__(256) void reduce_scatter_kernel(SpParts p, int64_t off4, int64_t nvec,
                                                             const f32x4* R, const uint32_t* __restrict__ keep,
                                                             float keep_prob, f32x4* out) {
  // out may be the residual itself (in-place update): each element is read and
  // then written by the same thread.
  const int64_t stride = (int64_t)gridDim.x * 256;
  for (int64_t v = (int64_t)blockIdx.x * 256 + threadIdx.x; v < nvec; v += stride) {
    f32x4 x[N];
#pragma unroll
    for (int i = 0; i < N; ++i) x[i] = __builtin_nontemporal_load(static_cast<const f32x4*>(p.p[i]) + off4 + v);
    f32x4 s = x[0];
#pragma unroll
    for (int i = 1; i < N; ++i) s = s + x[i];
    if (keep) {
      const uint32_t k = keep[v];
#pragma unroll
      for (int c = 0; c < 4; ++c) s[c] = ((k >> (8 * c)) & 0xffu) ? s[c] / keep_prob : 0.f;
    }
    if (R) s = __builtin_nontemporal_load(R + v) + s;
    __builtin_nontemporal_store(s, out + v);
  }
}

__global__ __launch_bounds__(256) void all_gather_kernel(SpParts p, int64_t nvec, u32x4* __restrict__ out) {
  const int j = blockIdx.y;
  const u32x4* src = static_cast<const u32x4*>(p.p[j]);
  u32x4* dst = out + (int64_t)j * nvec;
  const int64_t stride = (int64_t)gridDim.x * 256;
  for (int64_t v = (int64_t)blockIdx.x * 256 + threadIdx.x; v < nvec; v += stride)
    __builtin_nontemporal_store(__builtin_nontemporal_load(src + v), dst + v);
}

// Launches go(integral_constant<V>) for the smallest V of {1, 2, 3, 4, 6, 8, 12,
// 16, 24, 32} with vpt <= V <= VMAX (float4 per thread of a row workgroup).
template <int VMAX, int V = 1, typename F>
hipError_t pick_vpt(int vpt, F&& go) {
  if constexpr (V > VMAX) {
    return hipErrorInvalidValue;
  } else {
    if (vpt <= V) {
      go(std::integral_constant<int, V>{});
      return hipGetLastError();
    }
    constexpr int next = V < 4 ? V + 1 : (V % 3 == 0 ? V / 3 * 4 : V / 2 * 3);
    return pick_vpt<VMAX, next>(vpt, static_cast<F&&>(go));
  }
}

template <int N>
hipError_t launch_rs(const SpParts& p, int64_t off4, int64_t nvec, const float* R, const uint8_t* keep,
                     float keep_prob, float* out, hipStream_t st) {
  int64_t blocks = (nvec + 255) / 256;
  if (blocks > 256 * 8) blocks = 256 * 8;
  hipLaunchKernelGGL(reduce_scatter_kernel<N>, dim3((unsigned)blocks), dim3(256), 0, st, p, off4, nvec,
                     reinterpret_cast<const f32x4*>(R), reinterpret_cast<const uint32_t*>(keep), keep_prob,
                     reinterpret_cast<f32x4*>(out));
  return hipGetLastError();
}

}  // namespace

hipError_t layernorm_rows(const float* X, int64_t rows, int64_t h, const float* gamma, const float* beta, float eps,
                          uint16_t* Y, hipStream_t st) {
  if (rows == 0) return hipSuccess;
  const int64_t h4 = h / 4;
  const int vpt = (int)((h4 + kLnThreads - 1) / kLnThreads);
  const dim3 grid((unsigned)rows), block(kLnThreads);
  const float inv_h = 1.0f / (float)h;
  auto Xv = reinterpret_cast<const f32x4*>(X);
  auto Gv = reinterpret_cast<const f32x4*>(gamma);
  auto Bv = reinterpret_cast<const f32x4*>(beta);
  auto Yv = reinterpret_cast<uint2*>(Y);
  return pick_vpt<kLnMaxH / 4 / kLnThreads>(vpt, [&](auto vc) {
    hipLaunchKernelGGL((layernorm_kernel<decltype(vc)::value, kLnThreads>), grid, block, 0, st, Xv, h4, Gv, Bv, eps,
                       inv_h, Yv);
  });
}

hipError_t layernorm_bwd(const float* X, int64_t rows, int64_t h, const float* gamma, const float* dY,
                         const float* dRes, float eps, float* dX, float* dgamma, float* dbeta, void* ws,
                         hipStream_t st) {
  const int64_t h4 = h / 4;
  float2* stats = static_cast<float2*>(ws);
  float* pg = reinterpret_cast<float*>(static_cast<char*>(ws) + ((rows * 8 + 255) & ~int64_t(255)));
  float* pb = pg + kLnBwdRowBlocks * h;
  if (rows > 0) {
    const int vpt = (int)((h4 + kLnThreads - 1) / kLnThreads);
    const dim3 grid((unsigned)rows), block(kLnThreads);
    const float inv_h = 1.0f / (float)h;
    auto Xv = reinterpret_cast<const f32x4*>(X);
    auto Gv = reinterpret_cast<const f32x4*>(gamma);
    auto Dv = reinterpret_cast<const f32x4*>(dY);
    auto Rv = reinterpret_cast<const f32x4*>(dRes);
    auto Ov = reinterpret_cast<f32x4*>(dX);
    const hipError_t e = pick_vpt<kLnBwdMaxH / 4 / kLnThreads>(vpt, [&](auto vc) {
      hipLaunchKernelGGL((layernorm_bwd_rows_kernel<decltype(vc)::value, kLnThreads>), grid, block, 0, st, Xv, h4,
                         Gv, Dv, Rv, eps, inv_h, Ov, stats);
    });
    if (e != hipSuccess) return e;
  }
  const int nb = (int)(rows < kLnBwdRowBlocks ? (rows > 0 ? rows : 1) : kLnBwdRowBlocks);
  const int64_t rpb = rows > 0 ? (rows + nb - 1) / nb : 0;
  const unsigned gx = (unsigned)((h4 + 255) / 256);
  hipLaunchKernelGGL(layernorm_bwd_cols_kernel, dim3(gx, (unsigned)nb), dim3(256), 0, st,
                     reinterpret_cast<const f32x4*>(X), reinterpret_cast<const f32x4*>(dY), stats, rows, h4, rpb,
                     reinterpret_cast<f32x4*>(pg), reinterpret_cast<f32x4*>(pb));
  hipLaunchKernelGGL(colsum_kernel, dim3((unsigned)((h4 + 15) / 16)), dim3(256), 0, st, reinterpret_cast<const f32x4*>(pg),
                     reinterpret_cast<const f32x4*>(pb), nb, h4, reinterpret_cast<f32x4*>(dgamma),
                     reinterpret_cast<f32x4*>(dbeta));
  return hipGetLastError();
}

size_t layernorm_bwd_workspace(int64_t rows, int64_t h) {
  return (size_t)(((rows * 8 + 255) & ~int64_t(255)) + 2 * kLnBwdRowBlocks * h * 4);
}

hipError_t sp_dropout_bwd(const float* dY, int64_t rows, int64_t h, const uint8_t* keep, float keep_prob,
                          uint16_t* out, hipStream_t st) {
  const int64_t nvec = rows * h / 4;
  if (nvec == 0) return hipSuccess;
  int64_t blocks = (nvec + 255) / 256;
  if (blocks > 256 * 8) blocks = 256 * 8;
  hipLaunchKernelGGL(dropout_bwd_kernel, dim3((unsigned)blocks), dim3(256), 0, st, reinterpret_cast<const f32x4*>(dY),
                     reinterpret_cast<const uint32_t*>(keep), keep_prob, nvec, reinterpret_cast<uint2*>(out));
  return hipGetLastError();
}

hipError_t sp_reduce_scatter(const SpParts& parts, int n, int64_t row0, int64_t rows, int64_t h,
                             const float* residual, const uint8_t* keep, float keep_prob, float* out, hipStream_t st) {
  const int64_t nvec = rows * h / 4;
  if (nvec == 0) return hipSuccess;
  const int64_t off4 = row0 * h / 4;
  switch (n) {
#define TPS_CASE(k) \
  case k:           \
    return launch_rs<k>(parts, off4, nvec, residual, keep, keep_prob, out, st);
    TPS_CASE(1) TPS_CASE(2) TPS_CASE(3) TPS_CASE(4) TPS_CASE(5) TPS_CASE(6) TPS_CASE(7) TPS_CASE(8)
    TPS_CASE(9) TPS_CASE(10) TPS_CASE(11) TPS_CASE(12) TPS_CASE(13) TPS_CASE(14) TPS_CASE(15) TPS_CASE(16)
#undef TPS_CASE
    default:
      return hipErrorInvalidValue;
  }
}

hipError_t sp_all_gather(const SpParts& parts, int n, int64_t rows, int64_t h, uint16_t* out, hipStream_t st) {
  const int64_t nvec = rows * h / 8;
  if (nvec == 0 || n == 0) return hipSuccess;
  int64_t bx = (nvec + 255) / 256;
  const int64_t cap = (256 * 8 + n - 1) / n;
  if (bx > cap) bx = cap;
  hipLaunchKernelGGL(all_gather_kernel, dim3((unsigned)bx, (unsigned)n), dim3(256), 0, st, parts, nvec,
                     reinterpret_cast<u32x4*>(out));
  return hipGetLastError();
}

}  // namespace tps
