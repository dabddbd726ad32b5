// Host-side interface of the bf16 MFMA GEMM family (internal to libtpshard).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tps {

enum Epilogue { EPI_F32 = 0, EPI_BF16 = 1, EPI_GELU = 2, EPI_DGELU = 3, EPI_CE = 4 };

// Row statistics of the vocabulary-parallel cross-entropy kept by the EPI_CE
// epilogue, per row and per column slot: the slot's maximum logit and the sum of
// exp(logit - maximum) over the slot, as float32 (max, sum). A slot is half of a
// wave's 96-column block: in block b (columns 96b .. 96b+95), slot 2b + g holds
// the columns c with (c mod 32) / 16 == g. Columns at or beyond N are left out; a
// slot with none holds (-inf, 0). The target's logit is stored to ce_tlogit[m]
// for the rows whose target column lies in [0, N); other rows are not written.
constexpr int kCeBlock = 96;
__host__ __device__ inline int ce_slots(int N) { return 4 * (N / 192 + (N % 192 != 0)); }  // four per 192-wide tile

// C(m, n) = sum_k A(m, k) B(k, n).
//   A(m, k) = A[m * lda + k] when the A operand is K-contiguous, else A[k * lda + m].
//   B(k, n) = B[n * ldb + k] when the B operand is K-contiguous, else B[k * ldb + n].
// Epilogues: EPI_F32   C float32
//            EPI_BF16  C bf16
//            EPI_GELU  C bf16 = GeLU(acc); U (nullable) bf16 = acc
//            EPI_DGELU C bf16 = acc * GeLU'(Uin)
//            EPI_CE    C float32 [M][ce_slots(N)][2]: per row and column slot
//                      (max, sum exp(acc - max)); ce_tlogit[m] = acc(m, targets[m] - ce_lo)
//                      when that column lies in [0, N)
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
  // Stream-K workspace (nullable): when set and the last round of tiles fills at most
  // half of the persistent grid, the k-stages are split evenly over the workgroups and
  // the split tiles' float32 partials go here (kSkBytes, see gemm_bf16_sk_attach).
  float* sk_part = nullptr;
  // EPI_CE: row targets (vocabulary ids), the id of output column 0, and where the
  // targets' logits go.
  const int32_t* ce_targets = nullptr;
  int64_t ce_lo = 0;
  float* ce_tlogit = nullptr;
};

// Size of the stream-K area: two float32 256 x 192 tile slots per workgroup of the
// 256-workgroup grid.
constexpr size_t kSkBytes = (size_t)2 * 256 * 256 * 192 * 4;

// Workspace bytes a launch of an M x N x K product uses: kSkBytes when it runs
// stream-K (the last round of its 256 x 192 tiles fills at most half of the
// 256-workgroup grid; fewer than 1024 tiles; tiles of at least 48 k-stages), else 0.
size_t gemm_bf16_sk_workspace(int M, int N, int K);

// Points g's stream-K area at `area` (kSkBytes, 256-byte aligned), or clears it
// when the product does not run stream-K or area is null.
inline void gemm_bf16_sk_attach(GemmArgs& g, void* area) {
  g.sk_part = (area != nullptr && gemm_bf16_sk_workspace(g.M, g.N, g.K) != 0) ? static_cast<float*>(area) : nullptr;
}

hipError_t gemm_bf16(const GemmArgs& g, bool a_kcontig, bool b_kcontig, int epi, hipStream_t s);

}  // namespace tps
