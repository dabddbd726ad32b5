// bf16 MFMA GEMM family for gfx950: C[M,N] = sum_k A(m,k) B(k,n), float32
// accumulation in v_mfma_f32_32x32x16_bf16, with fused epilogues.
//
// One kernel template covers every product of the rank-shard MLP and attention:
//   operand layouts   A(m,k): K-contiguous ([M,K] row-major) or M-contiguous ([K,M])
//                     B(k,n): K-contiguous ([N,K] row-major) or N-contiguous ([K,N])
//   epilogues         float32 store | bf16 store | erf-GeLU (store U and GeLU(U) as
//                     bf16) | GeLU' (dU = acc * GeLU'(U) as bf16)
//
// Tiling: a 256-thread workgroup (4 waves, 2 x 2) owns a BM x BN tile of C and
// walks K in steps of BK = 64. Both operands are staged in LDS as [row][k] with
// k contiguous, 128 bytes per row, 16-byte chunks XOR-swizzled by the row so that
// the MFMA fragment reads (32 rows, same chunk) and the transposed stores (8 rows
// apart, same chunk) spread over all banks. LDS is double-buffered: the global
// loads of step t+1 are in flight in registers while the MFMAs of step t run;
// one barrier per step. Operands stored MN-contiguous are read as 8x8 blocks
// (8 k-rows x 16 bytes) and transposed in registers before the LDS store, so
// every global read is a coalesced 16-byte load.
//
// Workgroups are dispatched round-robin over the 8 XCDs; the tile index is
// remapped so each XCD owns a contiguous range of tiles (shared operand panels
// stay in that XCD's L2).
#include "common.hpp"
#include "gemm_bf16.hpp"

namespace tps {

namespace {

constexpr int BK = 64;          // k per LDS stage (128 bytes per row)
constexpr int NT = 256;         // threads per workgroup
constexpr int CHUNKS = BK / 8;  // 16-byte chunks per LDS row

__device__ __forceinline__ int swz(int row) { return (row ^ (row >> 3)) & 7; }

// Element offset of 16-byte chunk `kc` of LDS row `row`.
__device__ __forceinline__ int lds_off(int row, int kc) { return row * BK + ((kc ^ swz(row)) << 3); }

// ---------------------------------------------------------------- tile loaders
// K-contiguous source: element (r, k) at src[r * ld + k]. R rows x BK.
template <int R>
struct LoaderK {
  static constexpr int PER = R * CHUNKS / NT;  // 16-byte chunks per thread
  static_assert(R * CHUNKS % NT == 0, "tile rows must be a multiple of 32");
  u32x4 v[PER];

  __device__ __forceinline__ void load(const uint16_t* __restrict__ src, int64_t ld, int row0,
                                       int rows, int k0, int K, int tid) {
#pragma unroll
    for (int p = 0; p < PER; ++p) {
      const int c = tid + p * NT;
      const int r = c >> 3, kc = c & 7;
      const int gr = row0 + r, gk = k0 + kc * 8;
      if (gr < rows && gk < K)
        v[p] = *reinterpret_cast<const u32x4*>(src + (int64_t)gr * ld + gk);
      else
        v[p] = u32x4{0u, 0u, 0u, 0u};
    }
  }
  __device__ __forceinline__ void store(uint16_t* lds, int tid) const {
#pragma unroll
    for (int p = 0; p < PER; ++p) {
      const int c = tid + p * NT;
      const int r = c >> 3, kc = c & 7;
      *reinterpret_cast<u32x4*>(lds + lds_off(r, kc)) = v[p];
    }
  }
};

// MN-contiguous source: element (r, k) at src[k * ld + r]. Each active thread
// reads an 8(k) x 8(r) block as eight 16-byte row loads and transposes it.
template <int R>
struct LoaderMN {
  static constexpr int RB = R / 8;                    // 8-wide blocks along r
  static constexpr int NBLK = RB * CHUNKS;            // blocks per stage (= R)
  static constexpr int PER = (NBLK + NT - 1) / NT;    // blocks per thread
  static_assert(R % 8 == 0, "tile rows must be a multiple of 8");
  u32x4 v[PER][8];

  __device__ __forceinline__ void load(const uint16_t* __restrict__ src, int64_t ld, int row0,
                                       int rows, int k0, int K, int tid) {
#pragma unroll
    for (int p = 0; p < PER; ++p) {
      const int b = tid + p * NT;
      const int kb = b / RB, rb = b % RB;
      const int gr = row0 + rb * 8;
      const bool ok = (b < NBLK) && (gr < rows);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int gk = k0 + kb * 8 + j;
        if (ok && gk < K)
          v[p][j] = *reinterpret_cast<const u32x4*>(src + (int64_t)gk * ld + gr);
        else
          v[p][j] = u32x4{0u, 0u, 0u, 0u};
      }
    }
  }
  __device__ __forceinline__ void store(uint16_t* lds, int tid) const {
#pragma unroll
    for (int p = 0; p < PER; ++p) {
      const int b = tid + p * NT;
      if (b >= NBLK) break;
      const int kb = b / RB, rb = b % RB;
      // v[p][j] holds r = 0..7 of k-row j (two bf16 per dword). Row r of the
      // transposed block gathers element r of each of the 8 k-rows.
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        u32x4 lo, hi;  // r = 2q and r = 2q+1
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const uint32_t a = v[p][2 * w][q], c = v[p][2 * w + 1][q];
          lo[w] = (a & 0xffffu) | (c << 16);
          hi[w] = (a >> 16) | (c & 0xffff0000u);
        }
        const int r0 = rb * 8 + 2 * q;
        *reinterpret_cast<u32x4*>(lds + lds_off(r0, kb)) = lo;
        *reinterpret_cast<u32x4*>(lds + lds_off(r0 + 1, kb)) = hi;
      }
    }
  }
};

template <int R, bool KCONTIG>
struct LoaderSel;
template <int R>
struct LoaderSel<R, true> { using type = LoaderK<R>; };
template <int R>
struct LoaderSel<R, false> { using type = LoaderMN<R>; };

// ---------------------------------------------------------------- epilogue
// 32x32 accumulator layout: lane l, register e holds row 8*(e/4) + 4*(l/32) + e%4
// and column l%32 of the MFMA tile. `row0` already includes 4*(l/32), `col`
// the lane's column.
template <int EPI>
__device__ __forceinline__ void store_tile(const f32x16 a, const GemmArgs& g, int row0, int col) {
  if (col >= g.N) return;
  for (int e = 0; e < 16; ++e) {
    const int row = row0 + 8 * (e >> 2) + (e & 3);
    if (row >= g.M) continue;
    const float x = a[e];
    const int64_t o = (int64_t)row * g.ldc + col;
    if constexpr (EPI == EPI_F32) {
      static_cast<float*>(g.C)[o] = x;
    } else if constexpr (EPI == EPI_BF16) {
      static_cast<uint16_t*>(g.C)[o] = (uint16_t)f32_to_bf16_bits(x);
    } else if constexpr (EPI == EPI_GELU) {
      static_cast<uint16_t*>(g.C)[o] = (uint16_t)f32_to_bf16_bits(gelu_erf(x));
      if (g.U) g.U[(int64_t)row * g.ldu + col] = (uint16_t)f32_to_bf16_bits(x);
    } else {  // EPI_DGELU
      const float u = bf16_bits_to_f32(g.Uin[(int64_t)row * g.ldu + col]);
      static_cast<uint16_t*>(g.C)[o] = (uint16_t)f32_to_bf16_bits(x * gelu_erf_prime(u));
    }
  }
}

// ---------------------------------------------------------------- kernel
template <int BM, int BN, bool A_K, bool B_K, int EPI>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(1, 1)))
void gemm_bf16_kernel(GemmArgs g) {
  constexpr int WM = 2, WN = 2;                // wave grid
  constexpr int WTM = BM / WM, WTN = BN / WN;  // per-wave tile
  constexpr int TM = WTM / 32, TN = WTN / 32;  // 32x32 MFMA tiles per wave
  static_assert(WTM % 32 == 0 && WTN % 32 == 0, "wave tile must be a multiple of 32");

  __shared__ __attribute__((aligned(16))) uint16_t sA[2][BM * BK];
  __shared__ __attribute__((aligned(16))) uint16_t sB[2][BN * BK];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;

  // ---- tile index: XCD-contiguous remap, then column-major over tiles
  const int tiles_m = (g.M + BM - 1) / BM, tiles_n = (g.N + BN - 1) / BN;
  const int T = tiles_m * tiles_n;
  int w = blockIdx.x;
  {
    const int xcd = w & 7, idx = w >> 3, base = T >> 3, rem = T & 7;
    w = xcd * base + (xcd < rem ? xcd : rem) + idx;
  }
  const int tm = w % tiles_m, tn = w / tiles_m;
  const int m0 = tm * BM, n0 = tn * BN;

  typename LoaderSel<BM, A_K>::type la;
  typename LoaderSel<BN, B_K>::type lb;

  f32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  const int nk = (g.K + BK - 1) / BK;
  la.load(g.A, g.lda, m0, g.M, 0, g.K, tid);
  lb.load(g.B, g.ldb, n0, g.N, 0, g.K, tid);
  la.store(sA[0], tid);
  lb.store(sB[0], tid);
  __syncthreads();

  const int fr = lane & 31, fk = lane >> 5;  // fragment row, k-chunk parity
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) {
      la.load(g.A, g.lda, m0, g.M, (kt + 1) * BK, g.K, tid);
      lb.load(g.B, g.ldb, n0, g.N, (kt + 1) * BK, g.K, tid);
    }
    const uint16_t* a_s = sA[cur];
    const uint16_t* b_s = sB[cur];
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      bf16x8 af[TM], bfr[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i)
        af[i] = *reinterpret_cast<const bf16x8*>(a_s + lds_off(wm * WTM + i * 32 + fr, kk * 2 + fk));
#pragma unroll
      for (int j = 0; j < TN; ++j)
        bfr[j] = *reinterpret_cast<const bf16x8*>(b_s + lds_off(wn * WTN + j * 32 + fr, kk * 2 + fk));
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < nk) {
      la.store(sA[cur ^ 1], tid);
      lb.store(sB[cur ^ 1], tid);
    }
    __syncthreads();
  }

  // ---- epilogue
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
      store_tile<EPI>(acc[i][j], g, m0 + wm * WTM + i * 32 + 4 * fk, n0 + wn * WTN + j * 32 + fr);
}

template <int BM, int BN, bool A_K, bool B_K, int EPI>
hipError_t launch(const GemmArgs& g, hipStream_t s) {
  const int tiles = ((g.M + BM - 1) / BM) * ((g.N + BN - 1) / BN);
  if (tiles == 0) return hipSuccess;
  hipLaunchKernelGGL((gemm_bf16_kernel<BM, BN, A_K, B_K, EPI>), dim3(tiles), dim3(NT), 0, s, g);
  return hipGetLastError();
}

}  // namespace

hipError_t gemm_bf16(const GemmArgs& g, bool a_kcontig, bool b_kcontig, int epi, hipStream_t s) {
  constexpr int BM = 256, BN = 192;
  if (a_kcontig && !b_kcontig) {
    if (epi == EPI_GELU) return launch<BM, BN, true, false, EPI_GELU>(g, s);
    if (epi == EPI_BF16) return launch<BM, BN, true, false, EPI_BF16>(g, s);
    if (epi == EPI_F32) return launch<BM, BN, true, false, EPI_F32>(g, s);
  } else if (a_kcontig && b_kcontig) {
    if (epi == EPI_DGELU) return launch<BM, BN, true, true, EPI_DGELU>(g, s);
    if (epi == EPI_F32) return launch<BM, BN, true, true, EPI_F32>(g, s);
  } else if (!a_kcontig && !b_kcontig) {
    if (epi == EPI_F32) return launch<BM, BN, false, false, EPI_F32>(g, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace tps
