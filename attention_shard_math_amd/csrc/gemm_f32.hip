// float32 GEMM for the fp32 path of the column- and row-parallel linears:
// C[M,N] = X[M,K] W[K,N] with the same epilogues as the bf16 family (float32
// store, erf-GeLU with optional pre-activation store). Plain LDS-tiled FMA
// kernel: 64x64 tile per 256-thread workgroup, 4x4 outputs per thread, K in
// steps of 16. It serves small float32 shapes; the bf16 MFMA kernels carry
// the large ones.
#include "common.hpp"
#include "gemm_f32.hpp"

namespace tps {
namespace {

constexpr int TBM = 64, TBN = 64, TBK = 16;

template <bool GELU>
__global__ __launch_bounds__(256) void gemm_f32_kernel(const float* __restrict__ X, const float* __restrict__ W,
                                                       int M, int N, int K, float* __restrict__ C,
                                                       float* __restrict__ U) {
  __shared__ float sX[TBK][TBM + 1];
  __shared__ float sW[TBK][TBN + 1];
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
  const int m0 = blockIdx.y * TBM, n0 = blockIdx.x * TBN;
  float acc[4][4] = {};
  for (int k0 = 0; k0 < K; k0 += TBK) {
    for (int i = threadIdx.x; i < TBM * TBK; i += 256) {
      const int r = i / TBK, k = i % TBK;
      sX[k][r] = (m0 + r < M && k0 + k < K) ? X[(int64_t)(m0 + r) * K + k0 + k] : 0.f;
    }
    for (int i = threadIdx.x; i < TBK * TBN; i += 256) {
      const int k = i / TBN, c = i % TBN;
      sW[k][c] = (k0 + k < K && n0 + c < N) ? W[(int64_t)(k0 + k) * N + n0 + c] : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < TBK; ++k)
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(sX[k][ty * 4 + i], sW[k][tx * 4 + j], acc[i][j]);
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = m0 + ty * 4 + i;
    if (r >= M) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int c = n0 + tx * 4 + j;
      if (c >= N) continue;
      const int64_t o = (int64_t)r * N + c;
      if (GELU) {
        C[o] = gelu_erf(acc[i][j]);
        if (U) U[o] = acc[i][j];
      } else {
        C[o] = acc[i][j];
      }
    }
  }
}

}  // namespace

hipError_t gemm_f32(const float* X, const float* W, int M, int N, int K, float* C, float* U, bool gelu,
                    hipStream_t s) {
  if (M == 0 || N == 0) return hipSuccess;
  dim3 grid((N + TBN - 1) / TBN, (M + TBM - 1) / TBM);
  if (gelu)
    hipLaunchKernelGGL(gemm_f32_kernel<true>, grid, dim3(256), 0, s, X, W, M, N, K, C, U);
  else
    hipLaunchKernelGGL(gemm_f32_kernel<false>, grid, dim3(256), 0, s, X, W, M, N, K, C, U);
  return hipGetLastError();
}

}  // namespace tps
