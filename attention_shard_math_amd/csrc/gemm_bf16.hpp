// Host-side interface of the bf16 MFMA GEMM family (internal to libtpshard).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tps {

enum Epilogue { EPI_F32 = 0, EPI_BF16 = 1, EPI_GELU = 2, EPI_DGELU = 3 };

// C(m, n) = sum_k A(m, k) B(k, n).
//   A(m, k) = A[m * lda + k] when the A operand is K-contiguous, else A[k * lda + m].
//   B(k, n) = B[n * ldb + k] when the B operand is K-contiguous, else B[k * ldb + n].
// Epilogues: EPI_F32   C float32
//            EPI_BF16  C bf16
//            EPI_GELU  C bf16 = GeLU(acc); U (nullable) bf16 = acc
//            EPI_DGELU C bf16 = acc * GeLU'(Uin)
struct GemmArgs {
  const uint16_t* A;
  const uint16_t* B;
  int64_t lda, ldb;
  int M, N, K;
  void* C;
  int64_t ldc;
  uint16_t* U;          // EPI_GELU output (nullable)
  const uint16_t* Uin;  // EPI_DGELU input
  int64_t ldu;
};

hipError_t gemm_bf16(const GemmArgs& g, bool a_kcontig, bool b_kcontig, int epi, hipStream_t s);

}  // namespace tps
