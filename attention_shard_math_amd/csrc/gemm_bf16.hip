// bf16 MFMA GEMM family for gfx950: C[M,N] = sum_k A(m,k) B(k,n), float32
// accumulation in v_mfma_f32_32x32x16_bf16, with fused epilogues.
//
// One kernel template covers every product of the rank-shard MLP and attention:
//   operand layouts   A(m,k): K-contiguous ([M,K] row-major) or M-contiguous ([K,M])
//                     B(k,n): K-contiguous ([N,K] row-major) or N-contiguous ([K,N])
//   epilogues         float32 store | bf16 store | erf-GeLU (store U and GeLU(U) as
//                     bf16) | GeLU' (dU = acc * GeLU'(U) as bf16)
//
// Data path (no register staging): operand tiles go from HBM straight into LDS
// with buffer_load_dwordx4 ... lds, into a ring of NS stages of BK = 32 k-values;
// NS-1 stages are in flight while the MFMAs of the current one run. Each
// operand keeps its global orientation in LDS:
//   K-contiguous  -> LDS [row][k]  (64 bytes per row), fragments by ds_read_b128;
//   MN-contiguous -> LDS [k][row]  (2*R bytes per k), fragments by two
//                    ds_read_b64_tr_b16, which transpose 4x4 blocks of 16-bit
//                    values across each 16-lane group into the MFMA layout.
// A DMA lane always writes the next 16 LDS bytes of its wave's 1 KiB, so the
// bank swizzles below are applied by choosing which global chunk each lane
// fetches; both are conflict-free for the fragment reads.
//
// Workgroup: 768 threads = 12 waves for one BM x BN tile. Waves 0-7 only read
// LDS and issue MFMAs (a 4 x 2 grid of 64 x 96 wave tiles, the next k-step's
// fragments read while the current one's MFMAs run); waves 8-11 only issue the
// DMA of the ring and wait for it. A wave blocked issuing memory instructions
// (the texture unit accepts them at its own rate) thus never holds up the MFMA
// stream of its SIMD; each SIMD runs two MFMA waves and one DMA wave.
// The grid is persistent: 256 workgroups (one per CU; the LDS ring allows no
// more), each walking a list of tiles with the ring running on from one tile's
// last k-stage into the next tile's first, so the DMA of the next tile overlaps
// the current tile's epilogue instead of waiting for a new workgroup's launch.
// Workgroups are dispatched round-robin over the 8 XCDs; XCD x owns a contiguous
// range of tiles (in the grouped order of tile_rc), which its 32 workgroups take
// round-robin, so the operand panels they share stay in that XCD's L2.
#include "common.hpp"
#include "gemm_bf16.hpp"

namespace tps {

namespace {

typedef short s16x4 __attribute__((ext_vector_type(4)));
#define TPS_LDS(p) ((__attribute__((address_space(3))) void*)(p))

constexpr int BK = 32;                  // k per LDS stage
constexpr int NCW = 8;                  // MFMA waves (4 x 2 grid)
constexpr int NPW = 4;                  // DMA waves
constexpr int NT = 64 * (NCW + NPW);    // threads per workgroup
constexpr int NS = 5;                   // LDS ring depth
constexpr uint32_t kOOB = 0x7ffffff0u;  // buffer offset that reads as zero
constexpr int kGrid = 256;              // persistent grid: one workgroup per CU
constexpr int kBM = 256, kBN = 192;     // tile of every product

// Stream-K is used when the last round of tiles fills at most half of the grid,
// for fewer than four rounds of tiles (kSkMaxTiles), and for tiles of at least
// kSkMinStages k-stages.
// - With a fuller last round the split does not pay: the GEMMs run power-limited,
//   so the CUs that would idle mostly let the busy ones clock higher, while the
//   split adds the partials' traffic and a second kernel (measured: a 192-tile
//   product took 6% longer, a 264-tile one 5% less).
// - Each workgroup's run is a contiguous stretch of the tile order, so the 32 runs
//   side by side on an XCD sit a run's length apart in it and share few operand
//   panels in its L2, where the tile kernel deals an XCD consecutive tiles. The
//   longer the runs, the more that costs, while the last round's idle share
//   shrinks (measured: 2592 tiles took 1339 us with stream-K against 924 us in the
//   tile kernel, 864 tiles the same in both, 576 tiles 10% less with stream-K).
// - With tiles of fewer than kSkMinStages k-stages, a split tile's partials (192 KB
//   written and read back per piece) cost as much traffic as its operands
//   (measured: the per-head [4096, 4096] score products of an earlier 384-wide
//   attention backward, 12 stages per tile, made that backward 5% slower).
constexpr int kSkMaxTiles = 1023;
constexpr int kSkMinStages = 48;
__host__ __device__ constexpr bool sk_applies(int64_t tiles, int K) {
  return K >= kSkMinStages * BK && tiles > 0 && tiles % kGrid != 0 && tiles % kGrid <= kGrid / 2 &&
         tiles <= kSkMaxTiles && tiles * ((K + BK - 1) / BK) < (int64_t(1) << 30);
}

// s_waitcnt immediate that waits until at most n vector-memory operations are
// outstanding (expcnt and lgkmcnt left unconstrained): vmcnt in bits [3:0] and
// [15:14], expcnt [6:4], lgkmcnt [11:8].
constexpr int vmcnt_imm(int n) { return (n & 0xf) | (((n >> 4) & 3) << 14) | (0x7 << 4) | (0xf << 8); }

typedef int i32x4 __attribute__((ext_vector_type(4)));

// Raw buffer descriptor (stride 0): base address, size in bytes for the range
// check (reads past it return zero), and the default data format word.
__device__ __forceinline__ i32x4 make_rsrc(const void* p, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(p);
  return i32x4{(int)(uint32_t)a, (int)((a >> 32) & 0xffff), (int)bytes, 0x00020000};
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// ---- K-contiguous operand: LDS [row][k], 4 chunks of 16 bytes per row, so a
// 256-byte bank line holds 4 rows. Physical chunk = logical chunk ^ swk(row),
// swk(row) = (row / 4) % 4: the 16 rows of a 16-lane group then cover all 64
// banks once, and a fragment ds_read_b128 takes 4 LDS cycles. (Measured on
// gfx950 with the SQ_LDS_BANK_CONFLICT counter: 0 conflict cycles per read,
// against 4 for a swizzle built on rows {0,2,4,6} mod 8.)
__device__ __forceinline__ int swk(int row) { return (row >> 2) & 3; }
__device__ __forceinline__ int kc_off(int row, int c) { return row * BK + ((c ^ swk(row)) << 3); }

// ---- MN-contiguous operand: LDS [k][r], R/8 chunks per k-row. Physical chunk =
// logical chunk ^ mn_swz<R>(k). A transposing fragment read serves 32 lanes at a
// time: two 16-lane groups, each reading 32 bytes (2 chunks) of 4 consecutive
// k-rows, 4 consecutive chunks in all. With R = 192 a k-row is 384 bytes, so
// consecutive k-rows already fall half a bank line apart, and 2 * (k & 3) spreads
// the rest over distinct banks. With R = 256 a k-row is 512 bytes, two whole bank
// lines, so every k-row starts at the same bank. There 4 * (k & 3) places the 4
// k-rows' chunk quads on the 4 quarters of the 256-byte line (2 * (k & 3) put two
// k-rows on each chunk position: a 2-way conflict on every read, 0.8 conflict
// cycles per LDS instruction on the products with an M-contiguous A).
template <int R>
__device__ __forceinline__ int mn_swz(int k) {
  return (R % 256 == 0) ? (k & 3) << 2 : (k & 3) << 1;
}
template <int R>
__device__ __forceinline__ int mn_off(int k, int r) {
  return k * R + (((r >> 3) ^ mn_swz<R>(k)) << 3) + (r & 7);
}

// Issues the DMA of one stage of one operand. R = tile rows (M or N extent).
// Stage bytes = 64 * R = R/16 instructions of 1 KiB, split over the DMA waves.
template <int R, bool KCONTIG>
struct Dma {
  static constexpr int OPS = R / 16 / NPW;  // instructions per DMA wave per stage
  static_assert(R % 64 == 0 && (R / 16) % NPW == 0, "tile extent must be a multiple of 64");
  uint32_t base[OPS];  // per-lane element offset at k0 = 0 (kOOB if the row is out of range)
  int kofs[OPS];       // per-lane k offset inside the stage (for the k bound)

  __device__ __forceinline__ void init(int row0, int rows, int64_t ld, int wave, int lane) {
#pragma unroll
    for (int o = 0; o < OPS; ++o) {
      const int q = (wave * OPS + o) * 64 + lane;  // physical chunk inside the stage
      if constexpr (KCONTIG) {
        const int r = q >> 2, kc = (q & 3) ^ swk(r);
        kofs[o] = kc * 8;
        base[o] = (row0 + r < rows) ? (uint32_t)((int64_t)(row0 + r) * ld + kc * 8) : kOOB;
      } else {
        constexpr int CPR = R / 8;  // chunks per k-row
        static_assert(R % 256 == 0 || R % 64 == 0, "chunk swizzle must stay inside the k-row");
        const int k = q / CPR, c = (q % CPR) ^ mn_swz<R>(k);
        kofs[o] = k;
        base[o] = (row0 + c * 8 < rows) ? (uint32_t)((int64_t)k * ld + row0 + c * 8) : kOOB;
      }
    }
  }
  // k0: first k of the stage; ld: leading dimension (elements). The DMA is
  // issued as inline asm so the compiler's wait insertion does not treat it as
  // an LDS store it must wait for before every fragment read; completion is
  // awaited explicitly with s_waitcnt vmcnt before the stage barrier.
  __device__ __forceinline__ void issue(const i32x4& rs, uint32_t stage_lds, int64_t ld, int k0, int K,
                                        int wave) const {
#pragma unroll
    for (int o = 0; o < OPS; ++o) {
      const bool kok = k0 + kofs[o] < K;
      const int64_t add = KCONTIG ? (int64_t)k0 : (int64_t)k0 * ld;
      const uint32_t off = (base[o] != kOOB && kok) ? (uint32_t)((base[o] + add) * 2) : kOOB;
      const uint32_t dst = __builtin_amdgcn_readfirstlane(stage_lds + (uint32_t)((wave * OPS + o) * 1024));
      asm volatile("buffer_load_dwordx4 %0, %1, 0 offen lds" ::"v"(off), "s"(rs), "{m0}"(dst) : "memory");
    }
  }
};

// MFMA operand fragment for rows [rb, rb+32) of the tile and k-slice kk (16 k):
// lane l gets row rb + l%32 and k = 16*kk + 8*(l/32) + 0..7.
template <int R, bool KCONTIG>
__device__ __forceinline__ bf16x8 frag(const uint16_t* stage, int rb, int kk, int lane) {
  if constexpr (KCONTIG) {
    const int row = rb + (lane & 31);
    return *reinterpret_cast<const bf16x8*>(stage + kc_off(row, 2 * kk + (lane >> 5)));
  } else {
    const int g = lane >> 4, s = lane & 15;
    const int r = rb + 16 * (g & 1) + 4 * (s & 3);
    const int k = 16 * kk + 8 * (g >> 1) + (s >> 2);
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) s16x4*)(stage + mn_off<R>(k, r)));
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) s16x4*)(stage + mn_off<R>(k + 4, r)));
    const s16x4 v[2] = {lo, hi};
    return __builtin_bit_cast(bf16x8, v);
  }
}

// Tile t, in the order the workgroups walk them, -> tile row m and column n:
// groups of 4 tile-rows (all rows when their count is not a multiple of 4),
// column-major inside a group. The 32 tiles an XCD has in flight then form a
// 4 x 8 block, which fetches 4 A-panels of 256 rows and 8 B-panels of 192
// columns: 9% fewer bytes than the 8 x 4 block of plain column-major order.
__device__ __forceinline__ void tile_rc(int t, int tiles_m, int tiles_n, int& m, int& n) {
  const int gm = (tiles_m & 3) == 0 ? 4 : tiles_m;
  const int gs = gm * tiles_n, g = t / gs, l = t - g * gs;
  m = g * gm + l % gm;
  n = l / gm;
}

// ---------------------------------------------------------------- epilogue
// 32x32 accumulator layout: lane l, register e holds row 8*(e/4) + 4*(l/32) + e%4
// and column l%32 of the MFMA tile. `row0` already includes 4*(l/32), `col`
// the lane's column.
template <int EPI>
__device__ __forceinline__ void store_tile_scalar(const f32x16 a, const GemmArgs& g, int row0, int col) {
  if (col >= g.N) return;
  for (int e = 0; e < 16; ++e) {
    const int row = row0 + 8 * (e >> 2) + (e & 3);
    if (row >= g.M) continue;
    const float x = a[e];
    const int64_t o = (int64_t)row * g.ldc + col;
    if constexpr (EPI == EPI_F32) {
      __builtin_nontemporal_store(x, static_cast<float*>(g.C) + o);
    } else if constexpr (EPI == EPI_BF16) {
      static_cast<uint16_t*>(g.C)[o] = (uint16_t)f32_to_bf16_bits(x);
    } else if constexpr (EPI == EPI_GELU) {
      static_cast<uint16_t*>(g.C)[o] = (uint16_t)f32_to_bf16_bits(gelu_bf16out(x));
      if (g.U) g.U[(int64_t)row * g.ldu + col] = (uint16_t)f32_to_bf16_bits(x);
    } else {  // EPI_DGELU
      const float u = bf16_bits_to_f32(g.Uin[(int64_t)row * g.ldu + col]);
      static_cast<uint16_t*>(g.C)[o] = (uint16_t)f32_to_bf16_bits(x * gelu_prime_bf16out(u));
    }
  }
}

// Non-temporal (streaming) stores of the epilogues whose output is not read again
// by the next product (float32, bf16 and GeLU outputs): they leave the L2 to the
// operand panels the XCD's workgroups are still reading. Measured: the attention
// shard's QKV product 6% faster, the MLP products about 1%; the GeLU' output dU,
// which the next two products read, keeps ordinary stores.
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ void store_nt(uint16_t* p, uint32_t lo, uint32_t hi) {
  __builtin_nontemporal_store(u32x2{lo, hi}, reinterpret_cast<u32x2*>(p));
}

// Value of register x from lane (lane ^ 1) / (lane ^ 2) of the same quad.
__device__ __forceinline__ float quad_x1(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0xB1, 0xF, 0xF, true));
}
__device__ __forceinline__ float quad_x2(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x4E, 0xF, 0xF, true));
}

// Epilogue of one 32x32 accumulator tile. For the bf16 epilogues (GeLU, bf16,
// GeLU') on a whole in-range tile, each group of 4 registers (4 rows, one column
// per lane) is transposed across the lane quad, so that lane q of a quad holds row
// q and the quad's 4 consecutive columns: outputs are written (and GeLU' reads U)
// 8 bytes at a time instead of 2. (For the float32 store the per-element stores,
// 4 bytes each, measured faster.)
template <int EPI>
__device__ __forceinline__ void store_tile(const f32x16 a, const GemmArgs& g, int row0, int col, bool full) {
  if constexpr (EPI == EPI_DGELU || EPI == EPI_GELU || EPI == EPI_BF16) {
    if (full) {
      const int q = col & 3, c4 = col - q;
#pragma unroll
      for (int gr = 0; gr < 4; ++gr) {
        float v[4], t[4], w[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) v[j] = a[4 * gr + j];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float p = quad_x1(v[j ^ 1]);
          t[j] = ((q & 1) == (j & 1)) ? v[j] : p;
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float p = quad_x2(t[j ^ 2]);
          w[j] = (((q >> 1) & 1) == ((j >> 1) & 1)) ? t[j] : p;
        }
        const int row = row0 + 8 * gr + q;
        uint2* dst = reinterpret_cast<uint2*>(static_cast<uint16_t*>(g.C) + (int64_t)row * g.ldc + c4);
        if constexpr (EPI == EPI_DGELU) {
          const uint2 uu = *reinterpret_cast<const uint2*>(g.Uin + (int64_t)row * g.ldu + c4);
          const float u0 = bf16_bits_to_f32(uu.x & 0xffffu), u1 = bf16_bits_to_f32(uu.x >> 16);
          const float u2 = bf16_bits_to_f32(uu.y & 0xffffu), u3 = bf16_bits_to_f32(uu.y >> 16);
          *dst = uint2{pack_bf16x2(w[0] * gelu_prime_bf16out(u0), w[1] * gelu_prime_bf16out(u1)),
                       pack_bf16x2(w[2] * gelu_prime_bf16out(u2), w[3] * gelu_prime_bf16out(u3))};
        } else if constexpr (EPI == EPI_GELU) {
          store_nt(reinterpret_cast<uint16_t*>(dst), pack_bf16x2(gelu_bf16out(w[0]), gelu_bf16out(w[1])),
                   pack_bf16x2(gelu_bf16out(w[2]), gelu_bf16out(w[3])));
          if (g.U) store_nt(g.U + (int64_t)row * g.ldu + c4, pack_bf16x2(w[0], w[1]), pack_bf16x2(w[2], w[3]));
        } else {
          store_nt(reinterpret_cast<uint16_t*>(dst), pack_bf16x2(w[0], w[1]), pack_bf16x2(w[2], w[3]));
        }
      }
      return;
    }
  }
  store_tile_scalar<EPI>(a, g, row0, col);
}

// Reductions over the 16 lanes of each DPP row, every lane receiving the result:
// exchange with lane ^ 1 and lane ^ 2 (quad permutes), then with the mirrored lane
// of the half-row (i <-> 7 - i) and of the row (i <-> 15 - i). Each step combines
// two equal partials in either order, so all 16 lanes hold the same bits.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xf, 0xf, false));
}
constexpr int kDppXor1 = 0xB1, kDppXor2 = 0x4E, kDppHalfMirror = 0x141, kDppMirror = 0x140;
__device__ __forceinline__ float row16_sum(float x) {
  x += dpp_mov<kDppXor1>(x);
  x += dpp_mov<kDppXor2>(x);
  x += dpp_mov<kDppHalfMirror>(x);
  return x + dpp_mov<kDppMirror>(x);
}
__device__ __forceinline__ float row16_max(float x) {
  x = fmaxf(x, dpp_mov<kDppXor1>(x));
  x = fmaxf(x, dpp_mov<kDppXor2>(x));
  x = fmaxf(x, dpp_mov<kDppHalfMirror>(x));
  return fmaxf(x, dpp_mov<kDppMirror>(x));
}

// EPI_CE on one wave's 64 x 96 sub-tile at (r0, c0): the statistics of each row
// over each of the block's two column slots. The 16 lanes of a DPP row hold one
// row's values in a slot (lane l: row 8(e/4) + 4(l/32) + e%4 of each 32-row tile,
// column l%32 of each 32-column tile), so the slot reductions never leave the row.
// The exponentials are 2^(x log2(e) - max log2(e)) with the scaling in one fma
// (v_exp_f32 computes 2^x). The one lane that holds a row's target column stores
// its logit directly. WHOLE: every column of the block lies below N.
template <bool WHOLE, int TM, int TN>
__device__ __forceinline__ void ce_epilogue(const f32x16 (&acc)[TM][TN], const GemmArgs& g, int r0, int c0,
                                            int lane) {
  constexpr float kLog2e = 1.44269504088896340736f;
  constexpr float kNegInf = -__builtin_huge_valf();
  const int fk = lane >> 5, fr = lane & 31;
  const int nslot = ce_slots(g.N), slot = 2 * (c0 / kCeBlock) + (fr >> 4);
  f32x2* part = static_cast<f32x2*>(g.C);
#pragma unroll
  for (int i = 0; i < TM; ++i) {
    int tc[16];  // the rows' target columns (-1: not in this slice), fetched together
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int row = r0 + i * 32 + 8 * (e >> 2) + 4 * fk + (e & 3);
      const int64_t t = row < g.M ? (int64_t)g.ce_targets[row] - g.ce_lo : -1;
      tc[e] = t >= 0 && t < g.N ? (int)t : -1;
    }
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int row = r0 + i * 32 + 8 * (e >> 2) + 4 * fk + (e & 3);
      float x[TN];
#pragma unroll
      for (int j = 0; j < TN; ++j) x[j] = WHOLE || c0 + j * 32 + fr < g.N ? acc[i][j][e] : kNegInf;
      float mx = x[0];
#pragma unroll
      for (int j = 1; j < TN; ++j) mx = fmaxf(mx, x[j]);
      mx = row16_max(mx);
      // a slot with no column (only past N) has every x = -inf: scale by 0 instead
      const float mb = WHOLE ? mx * kLog2e : (mx == kNegInf ? 0.f : mx * kLog2e);
      float se = 0.f;
#pragma unroll
      for (int j = 0; j < TN; ++j) se += __builtin_amdgcn_exp2f(__builtin_fmaf(x[j], kLog2e, -mb));
      se = row16_sum(se);
      const int d = tc[e] - (c0 + fr);  // the target is this lane's column j when d == 32 j
#pragma unroll
      for (int j = 0; j < TN; ++j)
        if (d == 32 * j) g.ce_tlogit[row] = acc[i][j][e];
      if ((lane & 15) == 0 && row < g.M) part[(int64_t)row * nslot + slot] = f32x2{mx, se};
    }
  }
}

// Epilogue of one wave's 64 x 96 sub-tile at (r0, c0): per 32 x 32 tile for the
// stored epilogues, ce_epilogue for EPI_CE.
template <int EPI, int TM, int TN>
__device__ __forceinline__ void epilogue(const f32x16 (&acc)[TM][TN], const GemmArgs& g, int r0, int c0, int lane) {
  const int fk = lane >> 5, fr = lane & 31;
  if constexpr (EPI == EPI_CE) {
    static_assert(TN * 32 == kCeBlock, "one 96-column block per wave");
    // whole: no column of the block lies past N (every block but a slice's last)
    if (c0 + kCeBlock <= g.N)
      ce_epilogue<true>(acc, g, r0, c0, lane);
    else
      ce_epilogue<false>(acc, g, r0, c0, lane);
  } else {
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
        store_tile<EPI>(acc[i][j], g, r0 + i * 32 + 4 * fk, c0 + j * 32 + fr,
                        r0 + i * 32 + 32 <= g.M && c0 + j * 32 + 32 <= g.N);
  }
}

// ---------------------------------------------------------------- kernel
template <int BM, int BN, bool A_K, bool B_K, int EPI>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(3, 3)))
void gemm_bf16_kernel(GemmArgs g) {
  constexpr int WM = NCW / 2, WN = 2;          // MFMA wave grid
  constexpr int WTM = BM / WM, WTN = BN / WN;  // per-wave tile
  constexpr int TM = WTM / 32, TN = WTN / 32;  // 32x32 MFMA tiles per wave
  constexpr int SA = BM * BK, SB = BN * BK;    // stage sizes (elements)
  constexpr int DMA_OPS = (BM + BN) / 16 / NPW;  // DMA instructions per DMA wave per stage
  static_assert((NS - 2) * DMA_OPS < 64, "vmcnt range");
  static_assert(WTM % 32 == 0 && WTN % 32 == 0, "wave tile must be a multiple of 32");

  __shared__ __attribute__((aligned(1024))) uint16_t sA[NS][SA];
  __shared__ __attribute__((aligned(1024))) uint16_t sB[NS][SB];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;

  // ---- tile index: XCD-contiguous remap, then column-major over tiles
  const int tiles_m = (g.M + BM - 1) / BM, tiles_n = (g.N + BN - 1) / BN;
  const int T = tiles_m * tiles_n;
  // Persistent grid: XCD x (blockIdx % 8) owns a contiguous range of tiles, which its
  // workgroups take round-robin; the LDS ring runs on across a workgroup's tiles.
  const int per = gridDim.x >> 3, xcd = blockIdx.x & 7, jw = blockIdx.x >> 3;
  const int tbase = T >> 3, trem = T & 7;
  const int r0 = xcd * tbase + (xcd < trem ? xcd : trem), rn = tbase + (xcd < trem ? 1 : 0);
  const int ntl = jw < rn ? (rn - jw + per - 1) / per : 0;
  auto tile_m0 = [&](int i) {
    int m, n;
    tile_rc(r0 + jw + i * per, tiles_m, tiles_n, m, n);
    return m * BM;
  };
  auto tile_n0 = [&](int i) {
    int m, n;
    tile_rc(r0 + jw + i * per, tiles_m, tiles_n, m, n);
    return n * BN;
  };

  // Buffer resources cover each operand exactly; the host checks sizes < 2 GiB.
  const int64_t a_elems = A_K ? (int64_t)g.M * g.lda : (int64_t)g.K * g.lda;
  const int64_t b_elems = B_K ? (int64_t)g.N * g.ldb : (int64_t)g.K * g.ldb;
  const i32x4 ra = make_rsrc(g.A, (uint32_t)(a_elems * 2));
  const i32x4 rb = make_rsrc(g.B, (uint32_t)(b_elems * 2));

  const int nk = (g.K + BK - 1) / BK;
  const int total = ntl * nk;
  const uint32_t a_lds = lds_addr(&sA[0][0]), b_lds = lds_addr(&sB[0][0]);
  if (wave >= NCW) {
    // ---- DMA waves: stages 0 .. NS-2 in flight, then one refill per stage.
    const int pw = wave - NCW;
    Dma<BM, A_K> da;
    Dma<BN, B_K> db;
    // stages are issued in order: the next one's tile and k-stage are kept as counters
    int nti = 0, nkt = 0;
    auto issue_stage = [&](int gs, int sl) __attribute__((always_inline)) {
      (void)gs;
      if (nkt == 0) {
        da.init(tile_m0(nti), g.M, g.lda, pw, lane);
        db.init(tile_n0(nti), g.N, g.ldb, pw, lane);
      }
      da.issue(ra, a_lds + sl * SA * 2, g.lda, nkt * BK, g.K, pw);
      db.issue(rb, b_lds + sl * SB * 2, g.ldb, nkt * BK, g.K, pw);
      if (++nkt == nk) {
        nkt = 0;
        ++nti;
      }
    };
#pragma unroll
    for (int st = 0; st < NS - 1; ++st)
      if (st < total) issue_stage(st, st);
    int slot = 0;
    for (int t = 0; t < total; ++t) {
      // Stage t complete for this wave: at most the DMA of the later stages
      // already issued may be outstanding. The barrier then makes every DMA
      // wave's part visible, and tells that the MFMA waves are done with stage
      // t-1, whose slot is refilled below.
      const int after = min(t + NS - 2, total - 1) - t;
      if (after >= 3)
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(3 * DMA_OPS));
      else if (after == 2)
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * DMA_OPS));
      else if (after == 1)
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(DMA_OPS));
      else
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
      // A bare barrier: a workgroup fence would also wait for the later stages'
      // DMA. The empty asm keeps the compiler from moving memory ops across it.
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      if (t + NS - 1 < total) issue_stage(t + NS - 1, slot == 0 ? NS - 1 : slot - 1);
      slot = slot == NS - 1 ? 0 : slot + 1;
    }
    return;
  }

  // ---- MFMA waves
  const int am = wm * WTM, bn = wn * WTN;
  const int fk = lane >> 5, fr = lane & 31;
  int slot = 0;
  for (int it = 0; it < ntl; ++it) {
    f32x16 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;
    for (int t = 0; t < nk; ++t) {
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      const uint16_t* a_s = sA[slot];
      const uint16_t* b_s = sB[slot];
      constexpr int NKK = BK / 16;
      bf16x8 fa[2][TM], fb[2][TN];
#pragma unroll
      for (int i = 0; i < TM; ++i) fa[0][i] = frag<BM, A_K>(a_s, am + i * 32, 0, lane);
#pragma unroll
      for (int j = 0; j < TN; ++j) fb[0][j] = frag<BN, B_K>(b_s, bn + j * 32, 0, lane);
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) {
        const int cb = kk & 1;
        if (kk + 1 < NKK) {
#pragma unroll
          for (int i = 0; i < TM; ++i) fa[cb ^ 1][i] = frag<BM, A_K>(a_s, am + i * 32, kk + 1, lane);
#pragma unroll
          for (int j = 0; j < TN; ++j) fb[cb ^ 1][j] = frag<BN, B_K>(b_s, bn + j * 32, kk + 1, lane);
        }
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
          for (int j = 0; j < TN; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[cb][i], fb[cb][j], acc[i][j], 0, 0, 0);
      }
      slot = slot == NS - 1 ? 0 : slot + 1;
    }
    const int m0 = tile_m0(it), n0 = tile_n0(it);
    epilogue<EPI>(acc, g, m0 + am, n0 + bn, lane);
  }
}

// ---------------------------------------------------------------- stream-K
// Used when the last round of tiles would fill at most half of the 256
// workgroups (see sk_applies). The whole rounds (D = 256 * floor(T / 256) tiles,
// the first D of the order above) run as in the tile kernel: workgroup b takes
// tiles (b % 8) * D / 8 + b / 8 + 32 i, so an XCD works on consecutive tiles. The
// remaining (T - D) x nk (tile, k-stage) units are cut into 256 equal runs, one
// per workgroup (XCD-contiguous: workgroup b has virtual index
// v = (b % 8) * 32 + b / 8), which each workgroup takes after its whole tiles. A
// tile whose units all fall in one run is finished as in the tile kernel. For a
// tile split over several runs, each run writes its float32 accumulators to a
// workspace slot of its own (2 slots per run: its first and its last segment); a
// second kernel adds a split tile's partials in run order and runs the epilogue.
// No workgroup waits for another, and the sum order is fixed, so the result is
// reproducible.
template <int BM, int BN, bool A_K, bool B_K, int EPI>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(3, 3)))
void gemm_bf16_sk_kernel(GemmArgs g) {
  constexpr int WM = NCW / 2, WN = 2;
  constexpr int WTM = BM / WM, WTN = BN / WN;
  constexpr int TM = WTM / 32, TN = WTN / 32;
  constexpr int SA = BM * BK, SB = BN * BK;
  constexpr int DMA_OPS = (BM + BN) / 16 / NPW;
  constexpr int64_t SLOT = (int64_t)BM * BN / 4;  // float4 per workspace slot
  static_assert((NS - 2) * DMA_OPS < 64, "vmcnt range");

  __shared__ __attribute__((aligned(1024))) uint16_t sA[NS][SA];
  __shared__ __attribute__((aligned(1024))) uint16_t sB[NS][SB];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;

  const int tiles_m = (g.M + BM - 1) / BM, tiles_n = (g.N + BN - 1) / BN;
  const int nk = (g.K + BK - 1) / BK;
  const int G = gridDim.x;
  const int T = tiles_m * tiles_n, rounds = T / G, D = rounds * G;
  // whole tiles: workgroup b's i-th is xcd * D / 8 + jw + i * G / 8
  const int xcd = (int)(blockIdx.x & 7), jw = (int)(blockIdx.x >> 3);
  auto dp_tile = [&](int i) { return xcd * (D >> 3) + jw + i * (G >> 3); };
  // the remainder's units, tiles D .. T - 1 (the host keeps T * nk below 2^31)
  const int U = (T - D) * nk;
  const int v = xcd * (G >> 3) + jw;
  const int per = (U + G - 1) / G;
  const int g0 = min(U, v * per), g1 = min(U, g0 + per);
  const int whole = rounds * nk;  // units of this workgroup's whole tiles
  const int total = whole + (g1 - g0);
  auto tile_m0 = [&](int t) {
    int m, n;
    tile_rc(t, tiles_m, tiles_n, m, n);
    return m * BM;
  };
  auto tile_n0 = [&](int t) {
    int m, n;
    tile_rc(t, tiles_m, tiles_n, m, n);
    return n * BN;
  };
  // first remainder tile (counted from D) of run u (its slot 0 holds the partial of that tile)
  auto first_tile = [&](int u) { return u * per / nk; };

  const int64_t a_elems = A_K ? (int64_t)g.M * g.lda : (int64_t)g.K * g.lda;
  const int64_t b_elems = B_K ? (int64_t)g.N * g.ldb : (int64_t)g.K * g.ldb;
  const i32x4 ra = make_rsrc(g.A, (uint32_t)(a_elems * 2));
  const i32x4 rb = make_rsrc(g.B, (uint32_t)(b_elems * 2));
  const uint32_t a_lds = lds_addr(&sA[0][0]), b_lds = lds_addr(&sB[0][0]);

  if (wave >= NCW) {
    // ---- DMA waves: the same ring as the tile kernel, over this run's units. (The
    // ring and the stage body are written out in both kernels: a shared helper
    // taking the unit-to-tile mapping as a lambda compiled to slower DMA waves,
    // 2-3% on the MLP GEMMs, with bit-identical results.)
    const int pw = wave - NCW;
    Dma<BM, A_K> da;
    Dma<BN, B_K> db;
    int itile = -1;
    auto issue_stage = [&](int st, int sl) __attribute__((always_inline)) {
      int ti, kt;
      if (st < whole) {
        const int i = st / nk;
        ti = dp_tile(i);
        kt = st - i * nk;
      } else {
        const int gs = g0 + st - whole;
        ti = gs / nk;
        kt = gs - ti * nk;
        ti += D;
      }
      if (ti != itile) {
        da.init(tile_m0(ti), g.M, g.lda, pw, lane);
        db.init(tile_n0(ti), g.N, g.ldb, pw, lane);
        itile = ti;
      }
      da.issue(ra, a_lds + sl * SA * 2, g.lda, kt * BK, g.K, pw);
      db.issue(rb, b_lds + sl * SB * 2, g.ldb, kt * BK, g.K, pw);
    };
#pragma unroll
    for (int st = 0; st < NS - 1; ++st)
      if (st < total) issue_stage(st, st);
    int slot = 0;
    for (int t = 0; t < total; ++t) {
      const int after = min(t + NS - 2, total - 1) - t;
      if (after >= 3)
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(3 * DMA_OPS));
      else if (after == 2)
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * DMA_OPS));
      else if (after == 1)
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(DMA_OPS));
      else
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      if (t + NS - 1 < total) issue_stage(t + NS - 1, slot == 0 ? NS - 1 : slot - 1);
      slot = slot == NS - 1 ? 0 : slot + 1;
    }
    return;
  }

  // ---- MFMA waves: this workgroup's whole tiles, then one segment (a tile's
  // k-range inside this run) at a time.
  const int am = wm * WTM, bn = wn * WTN;
  const int fk = lane >> 5, fr = lane & 31;
  f32x4* part = reinterpret_cast<f32x4*>(g.sk_part);
  const int64_t wofs = (int64_t)wave * TM * TN * 4 * 64;  // this wave's float4 inside a slot
  int slot = 0;
  // k-stages [kb, ke) of one tile into acc (zeroed first), one ring slot per stage
  auto k_range = [&](f32x16 (&acc)[TM][TN], int kb, int ke) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;
    for (int t = kb; t < ke; ++t) {
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      const uint16_t* a_s = sA[slot];
      const uint16_t* b_s = sB[slot];
      constexpr int NKK = BK / 16;
      bf16x8 fa[2][TM], fb[2][TN];
#pragma unroll
      for (int i = 0; i < TM; ++i) fa[0][i] = frag<BM, A_K>(a_s, am + i * 32, 0, lane);
#pragma unroll
      for (int j = 0; j < TN; ++j) fb[0][j] = frag<BN, B_K>(b_s, bn + j * 32, 0, lane);
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) {
        const int cb = kk & 1;
        if (kk + 1 < NKK) {
#pragma unroll
          for (int i = 0; i < TM; ++i) fa[cb ^ 1][i] = frag<BM, A_K>(a_s, am + i * 32, kk + 1, lane);
#pragma unroll
          for (int j = 0; j < TN; ++j) fb[cb ^ 1][j] = frag<BN, B_K>(b_s, bn + j * 32, kk + 1, lane);
        }
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
          for (int j = 0; j < TN; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[cb][i], fb[cb][j], acc[i][j], 0, 0, 0);
      }
      slot = slot == NS - 1 ? 0 : slot + 1;
    }
  };
  for (int i = 0; i < rounds; ++i) {
    f32x16 acc[TM][TN];
    k_range(acc, 0, nk);
    const int ti = dp_tile(i);
    epilogue<EPI>(acc, g, tile_m0(ti) + am, tile_n0(ti) + bn, lane);
  }
  int gs = g0;
  while (gs < g1) {
    const int ti = gs / nk;  // counted from D
    const int kb = gs - ti * nk;
    const int ke = min(nk, g1 - ti * nk);
    f32x16 acc[TM][TN];
    k_range(acc, kb, ke);
    const bool split = kb != 0 || ke != nk;
    if (split) {
      // This run's share of a split tile: to its slot, in accumulator order.
      f32x4* mine = part + (2LL * v + (ti == first_tile(v) ? 0 : 1)) * SLOT + wofs;
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
          for (int q = 0; q < 4; ++q)
            mine[((i * TN + j) * 4 + q) * 64 + lane] =
                f32x4{acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]};
    }
    if (!split) epilogue<EPI>(acc, g, tile_m0(D + ti) + am, tile_n0(D + ti) + bn, lane);
    gs = ti * nk + ke;
  }
}

// Finishes the split tiles of a stream-K launch. The remainder tiles (D .. T - 1)
// are summed in 32-row blocks of the MFMA waves' sub-tiles: workgroup
// (8 t + w) TM + i is one wave laid out like MFMA wave w of the product kernel (the
// same accumulator tiles per lane), adds row block i of that wave's share of the
// partials of the runs covering tile D + t in run order, and runs the same epilogue
// on it. The blocks are independent (the cross-entropy statistics are per row), and
// a few tiles cut into many pieces are read by as many single-wave workgroups as
// possible, since each wave's sum is bound by its loads' latency. Workgroups of
// tiles that one run finished exit at once.
template <int BM, int BN, int EPI>
__global__ __launch_bounds__(64) void gemm_bf16_sk_fixup_kernel(GemmArgs g) {
  constexpr int WM = NCW / 2, WN = 2;
  constexpr int WTM = BM / WM, WTN = BN / WN;
  constexpr int TM = WTM / 32, TN = WTN / 32;
  constexpr int64_t SLOT = (int64_t)BM * BN / 4;
  const int lane = threadIdx.x;
  const int i = blockIdx.x % TM, wave = (blockIdx.x / TM) % NCW;
  const int ti = blockIdx.x / (TM * NCW);  // counted from D
  const int wm = wave / WN, wn = wave % WN;
  const int tiles_m = (g.M + BM - 1) / BM, tiles_n = (g.N + BN - 1) / BN;
  const int nk = (g.K + BK - 1) / BK;
  const int T = tiles_m * tiles_n, D = T / kGrid * kGrid;
  const int U = (T - D) * nk;
  const int per = (U + kGrid - 1) / kGrid;
  const int ua = ti * nk;
  const int vf = ua / per, vl = (ua + nk - 1) / per;
  if (vf == vl) return;
  const f32x4* part = reinterpret_cast<const f32x4*>(g.sk_part);
  const int64_t bofs = ((int64_t)wave * TM + i) * TN * 4 * 64;
  f32x16 acc[1][TN];
  // The partials are loaded FG pieces at a time before they are added, so a tile cut
  // into many pieces waits for one load latency per group rather than per piece.
  // The sum is still ((P_vf + P_vf+1) + ...) in run order.
  constexpr int FG = 4;
  for (int u0 = vf; u0 <= vl; u0 += FG) {
    f32x4 x[FG][TN][4];
#pragma unroll
    for (int gi = 0; gi < FG; ++gi)
      if (u0 + gi <= vl) {
        const int u = u0 + gi;
        const f32x4* src = part + (2LL * u + (ti == u * per / nk ? 0 : 1)) * SLOT + bofs;
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
          for (int q = 0; q < 4; ++q) x[gi][j][q] = src[(j * 4 + q) * 64 + lane];
      }
#pragma unroll
    for (int gi = 0; gi < FG; ++gi)
      if (u0 + gi <= vl) {
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
          for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int r = 0; r < 4; ++r)
              acc[0][j][4 * q + r] = u0 + gi == vf ? x[gi][j][q][r] : acc[0][j][4 * q + r] + x[gi][j][q][r];
      }
  }
  int tm, tn;
  tile_rc(D + ti, tiles_m, tiles_n, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;
  const int am = wm * WTM + i * 32, bn = wn * WTN;
  epilogue<EPI>(acc, g, m0 + am, n0 + bn, lane);
}

template <int BM, int BN, bool A_K, bool B_K, int EPI>
hipError_t launch(const GemmArgs& g, hipStream_t s) {
  const int tiles = ((g.M + BM - 1) / BM) * ((g.N + BN - 1) / BN);
  if (tiles == 0) return hipSuccess;
  if (g.sk_part && sk_applies(tiles, g.K)) {
    hipLaunchKernelGGL((gemm_bf16_sk_kernel<BM, BN, A_K, B_K, EPI>), dim3(kGrid), dim3(NT), 0, s, g);
    // one single-wave workgroup per (remainder tile, MFMA wave, 32-row block)
    constexpr int fix_per_tile = NCW * (BM / (NCW / 2) / 32);
    hipLaunchKernelGGL((gemm_bf16_sk_fixup_kernel<BM, BN, EPI>), dim3((tiles % kGrid) * fix_per_tile), dim3(64), 0, s,
                       g);
    return hipGetLastError();
  }
  // one workgroup per CU (the LDS ring allows no more), a multiple of 8 for the XCD split
  const int grid = tiles >= kGrid ? kGrid : ((tiles + 7) & ~7);
  hipLaunchKernelGGL((gemm_bf16_kernel<BM, BN, A_K, B_K, EPI>), dim3(grid), dim3(NT), 0, s, g);
  return hipGetLastError();
}

}  // namespace

size_t gemm_bf16_sk_workspace(int M, int N, int K) {
  const int64_t tiles = (int64_t)((M + kBM - 1) / kBM) * ((N + kBN - 1) / kBN);
  return sk_applies(tiles, K) ? kSkBytes : 0;
}

hipError_t gemm_bf16(const GemmArgs& g, bool a_kcontig, bool b_kcontig, int epi, hipStream_t s) {
  constexpr int BM = kBM, BN = kBN;
  // buffer loads address each operand with 32-bit byte offsets
  const int64_t a_bytes = 2 * (a_kcontig ? (int64_t)g.M * g.lda : (int64_t)g.K * g.lda);
  const int64_t b_bytes = 2 * (b_kcontig ? (int64_t)g.N * g.ldb : (int64_t)g.K * g.ldb);
  if (a_bytes >= (int64_t)kOOB || b_bytes >= (int64_t)kOOB) return hipErrorInvalidValue;
  if (a_kcontig && !b_kcontig) {
    if (epi == EPI_GELU) return launch<BM, BN, true, false, EPI_GELU>(g, s);
    if (epi == EPI_BF16) return launch<BM, BN, true, false, EPI_BF16>(g, s);
    if (epi == EPI_F32) return launch<BM, BN, true, false, EPI_F32>(g, s);
  } else if (a_kcontig && b_kcontig) {
    if (epi == EPI_DGELU) return launch<BM, BN, true, true, EPI_DGELU>(g, s);
    if (epi == EPI_CE) return launch<BM, BN, true, true, EPI_CE>(g, s);
    if (epi == EPI_F32) return launch<BM, BN, true, true, EPI_F32>(g, s);
    if (epi == EPI_BF16) return launch<BM, BN, true, true, EPI_BF16>(g, s);
  } else if (!a_kcontig && !b_kcontig) {
    if (epi == EPI_F32) return launch<BM, BN, false, false, EPI_F32>(g, s);
    if (epi == EPI_BF16) return launch<BM, BN, false, false, EPI_BF16>(g, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace tps
