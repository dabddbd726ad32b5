// Host-side interface of the float32 GEMM (internal to libtpshard).
#pragma once
#include <hip/hip_runtime.h>

namespace tps {
// C[M,N] = X[M,K] W[K,N], all row-major float32. With gelu: C = GeLU(XW) and,
// if U is not null, U = XW.
hipError_t gemm_f32(const float* X, const float* W, int M, int N, int K, float* C, float* U, bool gelu,
                    hipStream_t s);
}  // namespace tps
