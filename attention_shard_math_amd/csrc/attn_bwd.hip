// Backward of the fused causal attention (gfx950), deterministic, no atomics.
//
// With P = exp(S/sqrt(d) - lse) recomputed from the forward's log-sum-exp:
//   dV = P^T dO,  dP = dO V^T,  dS = P * (dP - D),  D = rowsum(dO * O),
//   dQ = dS K / sqrt(d),  dK = dS^T Q / sqrt(d).
// Three launches:
//   * rowdot — D per (query, head), 16 lanes per row of 128;
//   * dkdv_dq — one grid holding the two independent walks, dK/dV items first,
//     so that dQ items start on the CUs the dK/dV tail leaves free:
//     - a dK/dV item is one workgroup per (sequence, head, block of 32*NW keys),
//       wave w owning 32 keys (their K and V fragments, dK and dV in
//       registers); it walks the query blocks of 32 that can see its keys, with
//       each block's Q and dO staged in LDS (double-buffered) and shared by the
//       waves;
//     - a dQ item is one workgroup per (sequence, head, block of 32*NW
//       queries), wave w owning 32 queries whose Q and dO fragments sit in
//       registers; it walks the key blocks of 32 up to the diagonal, K and V
//       staged in LDS;
//   * combine — the walks are cut into chunks for causal balance, and this
//     launch adds the chunks' partials of dQ, dK and dV in chunk order.
// The staged tiles are loaded into registers two steps ahead of their use (two
// register sets, the loop unrolled by two), so a step's compute covers the
// global-load latency of the tile after next.
// Both walks run their products on v_mfma_f32_32x32x16_bf16. The score
// tile comes out of the MFMA with a lane owning one column and 16 rows
// {8(e/4) + 4(l/32) + e%4}; those 16 values (8 per 16-row k-slice, packed to
// bf16) are used directly as the k-operand of the next product, taking the
// k-slice in that permuted order. The other operand of that product is read
// from LDS with ds_read_b64_tr_b16, whose 4-row groups are picked to match
// the same order, so no score tile goes through LDS.
//
// P and dS enter the products dV = P^T dO, dK = dS^T Q and dQ = dS K as two
// bf16 MFMA operands each, hi = bf16(x) and lo = bf16(x - hi), so they carry
// about 16 significant bits instead of 8. The bf16-stored dQ, dK, dV then round
// to the same value as the exact gradient in all but a small fraction of
// entries, which keeps the weight gradients formed from them (X^T dQKV over
// thousands of tokens) within the bf16 bar.
//
// LDS rows hold one head's d columns; 16-byte chunk c of row r is stored at
// c ^ swz(r), swz(r) = ((r & 7) << 1) | ((r >> 3) & 1), conflict-free for the
// 16-row ds_read_b128 fragment reads (384-wide rows use swz384, inside each group
// of 16 chunks).
//
// Heads of d = 384 take the same walks with the work of a step split over four
// waves (see dkdv_wide_item).
#include <type_traits>

#include "attn.hpp"
#include "common.hpp"


namespace tps {
namespace {

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ int swz(int r) { return ((r & 7) << 1) | ((r >> 3) & 1); }

// Element offset of (row r, column c) in a [rows][D] bf16 LDS tile (c % 4 == 0
// for transposing reads; any c inside its 16-byte chunk).
// Chunk swizzle of the 384-wide tiles: a permutation of the row's low 4 bits, so
// that 16 consecutive rows take 16 distinct chunk positions (the ds_read_b128
// fragment reads) and 4 consecutive rows 4 distinct aligned groups of 4 positions
// (the 4-row x 4-chunk transposing reads, which swz gives 2-way bank conflicts).
__device__ __forceinline__ int swz384(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }

template <int D>
__device__ __forceinline__ int toff(int r, int c) {
  if constexpr (D == 384)  // 48 chunks a row: the xor (< 16) stays inside each group of 16
    return r * D + (((c >> 3) ^ swz384(r)) << 3) + (c & 7);
  else
    return r * D + ((((c >> 3) ^ swz(r)) & (D / 8 - 1)) << 3) + (c & 7);
}

// ds_read_b128 fragment: lane gets row rb + l%32, columns 16kk + 8(l/32) .. +8.
template <int D>
__device__ __forceinline__ bf16x8 frag_rows(const uint16_t* t, int rb, int kk, int lane) {
  return *reinterpret_cast<const bf16x8*>(t + toff<D>(rb + (lane & 31), 16 * kk + 8 * (lane >> 5)));
}

// Transposing fragment of a [k][n] tile for the k-operand order of a score
// tile: lane gets column nb + l%32 and rows kb + {4h + 0..3, 8 + 4h + 0..3},
// h = l/32 (the rows the score accumulator gives that lane in registers e, e+4..).
template <int D>
__device__ __forceinline__ bf16x8 frag_tr(const uint16_t* t, int kb, int nb, int lane) {
  const int g = lane >> 4, sl = lane & 15;
  const int k = kb + 4 * (g >> 1) + (sl >> 2);
  const int n = nb + 16 * (g & 1) + 4 * (sl & 3);
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(t + toff<D>(k, n)));
  const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(t + toff<D>(k + 8, n)));
  const s16x4 v[2] = {lo, hi};
  return __builtin_bit_cast(bf16x8, v);
}


// Score registers e0..e0+7 as a bf16 k-operand.
__device__ __forceinline__ bf16x8 pack8(const float* v) {
  u32x4 u;
#pragma unroll
  for (int w = 0; w < 4; ++w) u[w] = pack_bf16x2(v[2 * w], v[2 * w + 1]);
  return __builtin_bit_cast(bf16x8, u);
}

// Residual of pack8: bf16(v - hi) for the values whose bf16 rounding is hi.
__device__ __forceinline__ bf16x8 pack8_lo(const float* v, bf16x8 hi) {
  const u32x4 h = __builtin_bit_cast(u32x4, hi);
  u32x4 u;
#pragma unroll
  for (int w = 0; w < 4; ++w)
    u[w] = pack_bf16x2(v[2 * w] - bf16_bits_to_f32(h[w] & 0xffffu), v[2 * w + 1] - bf16_bits_to_f32(h[w] >> 16));
  return __builtin_bit_cast(bf16x8, u);
}

// Stage rows [r0, r0 + R) of one head's D columns of a [rows][ld] bf16 tensor
// into a swizzled [R][D] LDS tile; rows at or past `rows` are zero.
template <int D, int R, int NTH>
__device__ __forceinline__ void load_rows(u32x4 (&reg)[R * D / 8 / NTH], const uint16_t* g, int64_t ld, int r0,
                                          int rows, int tid) {
  constexpr int CPR = D / 8;
#pragma unroll
  for (int p = 0; p < R * D / 8 / NTH; ++p) {
    const int c = tid + p * NTH, r = c / CPR, ch = c % CPR;
    reg[p] = (r0 + r < rows) ? *reinterpret_cast<const u32x4*>(g + (int64_t)(r0 + r) * ld + ch * 8)
                             : u32x4{0u, 0u, 0u, 0u};
  }
}
template <int D, int R, int NTH>
__device__ __forceinline__ void store_rows(const u32x4 (&reg)[R * D / 8 / NTH], uint16_t* t, int tid) {
  constexpr int CPR = D / 8;
#pragma unroll
  for (int p = 0; p < R * D / 8 / NTH; ++p) {
    const int c = tid + p * NTH, r = c / CPR, ch = c % CPR;
    *reinterpret_cast<u32x4*>(t + toff<D>(r, ch * 8)) = reg[p];
  }
}

// ------------------------------------------------------------------ D = rowsum(dO * O)
__global__ __launch_bounds__(256) void rowdot_kernel(const uint16_t* __restrict__ dO, const uint16_t* __restrict__ O,
                                                     float* __restrict__ Dout, int s, int Hl, int D, int64_t rows) {
  const int64_t r = (int64_t)blockIdx.x * 16 + (threadIdx.x >> 4);  // (token, head)
  const int j0 = threadIdx.x & 15;
  const int cpr = D / 8;  // 16-byte chunks per head row (8, 16 or 48)
  float acc = 0.f;
  if (r < rows) {
    const int64_t t = r / Hl, head = r % Hl;
    for (int j = j0; j < cpr; j += 16) {
      const int64_t off = t * (int64_t)Hl * D + head * D + j * 8;
      const u32x4 a = *reinterpret_cast<const u32x4*>(dO + off);
      const u32x4 b = *reinterpret_cast<const u32x4*>(O + off);
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        acc += bf16_bits_to_f32(a[w] & 0xffffu) * bf16_bits_to_f32(b[w] & 0xffffu);
        acc += bf16_bits_to_f32(a[w] >> 16) * bf16_bits_to_f32(b[w] >> 16);
      }
    }
  }
#pragma unroll
  for (int o = 8; o > 0; o >>= 1) acc += __shfl_xor(acc, o, 16);
  if (r < rows && j0 == 0) {
    const int64_t t = r / Hl, head = r % Hl, bi = t / s, q = t % s;
    Dout[(bi * Hl + head) * s + q] = acc;
  }
}

// ------------------------------------------------------------------ causal balance
// A block's walk of n steps (32 rows each) is cut into ceil(n / C) chunks of at
// most C steps, each run by its own workgroup, so the diagonal blocks' long walks
// no longer set the kernel's length. A chunk of a block that has several writes
// its fp32 partial to a workspace slot; combine_kernel adds a block's partials in
// chunk order afterwards (deterministic). C is chosen so that no block has more
// than kMaxChunks chunks.
constexpr int kMaxChunks = 4;

// Steps of key block kb's walk over query blocks (dK, dV).
template <bool CAUSAL>
__device__ __host__ __forceinline__ int kv_steps(int kb, int KB, int s) {
  return (s - (CAUSAL ? kb * KB : 0) + 31) / 32;
}
// Steps of query block qb's walk over key blocks (dQ).
template <bool CAUSAL>
__device__ __host__ __forceinline__ int q_steps(int qb, int QB, int s) {
  return ((CAUSAL ? min(s, (qb + 1) * QB) : s) + 31) / 32;
}

// Rank r of a head's chunks (0 = the heaviest block's first chunk) -> (block, chunk).
template <bool CAUSAL, bool QSIDE>
__device__ __forceinline__ void chunk_of(int r, int nblk, int R, int s, int C, int& blk, int& c) {
  for (int i = 0; i < nblk; ++i) {
    const int b = QSIDE ? nblk - 1 - i : i;  // causal: the last query block / first key block is heaviest
    const int n = (QSIDE ? q_steps<CAUSAL>(b, R, s) : kv_steps<CAUSAL>(b, R, s));
    const int nc = (n + C - 1) / C;
    if (r < nc) {
      blk = b;
      c = r;
      return;
    }
    r -= nc;
  }
  blk = -1;
  c = 0;
}

// out[row, col0 + d] = bf16(scale * sum_c part[c][row][d]) for every block with
// more than one chunk. part slots: [bh][blk][kMaxChunks][R][D] float32.
template <int D, bool CAUSAL, bool QSIDE>
__device__ __forceinline__ void combine_part(const float* __restrict__ part, uint16_t* __restrict__ out, int s,
                                             int Hl, int nblk, int R, int C, int col_block, float scale) {
  const int bh = blockIdx.x / nblk, blk = blockIdx.x % nblk;
  const int n = QSIDE ? q_steps<CAUSAL>(blk, R, s) : kv_steps<CAUSAL>(blk, R, s);
  const int nc = (n + C - 1) / C;
  if (nc <= 1) return;
  const int bi = bh / Hl, head = bh % Hl;
  const int64_t ld = 3LL * Hl * D;
  const float* pb = part + ((int64_t)bh * nblk + blk) * kMaxChunks * R * D;
  for (int v = blockIdx.y * 256 + threadIdx.x; v < R * D / 4; v += gridDim.y * 256) {
    const int row = blk * R + (v * 4) / D, d = (v * 4) % D;
    if (row >= s) continue;
    f32x4 a = *reinterpret_cast<const f32x4*>(pb + (int64_t)v * 4);
    for (int c = 1; c < nc; ++c) a = a + *reinterpret_cast<const f32x4*>(pb + (int64_t)c * R * D + v * 4);
    uint2 u;
    u.x = pack_bf16x2(a[0] * scale, a[1] * scale);
    u.y = pack_bf16x2(a[2] * scale, a[3] * scale);
    *reinterpret_cast<uint2*>(out + ((int64_t)bi * s + row) * ld + (int64_t)(col_block * Hl + head) * D + d) = u;
  }
}

// blockIdx.z: 0 = dQ (scaled), 1 = dK (scaled), 2 = dV; one launch for the three.
template <int D, bool CAUSAL>
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ partQ,
                                                      const float* __restrict__ partK,
                                                      const float* __restrict__ partV, uint16_t* __restrict__ out,
                                                      int s, int Hl, int nblk, int R, int C, float scale) {
  if (blockIdx.z == 0)
    combine_part<D, CAUSAL, true>(partQ, out, s, Hl, nblk, R, C, 0, scale);
  else
    combine_part<D, CAUSAL, false>(blockIdx.z == 1 ? partK : partV, out, s, Hl, nblk, R, C, (int)blockIdx.z,
                                   blockIdx.z == 1 ? scale : 1.f);
}

// ------------------------------------------------------------------ dK, dV
template <int D, bool CAUSAL, int NW>
__device__ __forceinline__ void dkdv_item(int item, const uint16_t* __restrict__ qkv,
                                                       const uint16_t* __restrict__ dO,
                                                       const float* __restrict__ lse,
                                                       const float* __restrict__ Dv, uint16_t* __restrict__ dqkv,
                                                       float* __restrict__ partK, float* __restrict__ partV, int s,
                                                       int Hl, int BH, int nkb, int C, float scale_log2,
                                                       float scale) {
  constexpr int NTH = NW * 64, KB = 32 * NW, KS = D / 16, DT = D / 32;
  constexpr int QP = 32 * D / 8 / NTH;  // 16-byte chunks per thread per 32-row tile
  __shared__ __attribute__((aligned(16))) uint16_t sK[KB * D];
  __shared__ __attribute__((aligned(16))) uint16_t sV[KB * D];
  __shared__ __attribute__((aligned(16))) uint16_t sQ[2][32 * D];
  __shared__ __attribute__((aligned(16))) uint16_t sdO[2][32 * D];
  __shared__ __attribute__((aligned(16))) float sL[2][32];
  __shared__ __attribute__((aligned(16))) float sDv[2][32];

  // Chunks of every head, heaviest first: rank r of all heads before rank r + 1.
  const int bh = item % BH;
  int kb, chunk;
  chunk_of<CAUSAL, false>(item / BH, nkb, KB, s, C, kb, chunk);
  if (kb < 0) return;
  const int bi = bh / Hl, head = bh % Hl;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, lr = lane & 31, hh = lane >> 5;
  const int64_t ld = 3LL * Hl * D, ldo = (int64_t)Hl * D;
  const uint16_t* Qg = qkv + (int64_t)bi * s * ld + (int64_t)head * D;
  const uint16_t* Kg = Qg + (int64_t)Hl * D;
  const uint16_t* Vg = Qg + 2LL * Hl * D;
  const uint16_t* dOg = dO + (int64_t)bi * s * ldo + (int64_t)head * D;
  const float* lseg = lse + (int64_t)bh * s;
  const float* Dg = Dv + (int64_t)bh * s;
  const int k0 = kb * KB, kw = k0 + 32 * wave;

  {
    constexpr int KP = KB * D / 8 / NTH;
    u32x4 r[KP];
    load_rows<D, KB, NTH>(r, Kg, ld, k0, s, tid);
    store_rows<D, KB, NTH>(r, sK, tid);
    load_rows<D, KB, NTH>(r, Vg, ld, k0, s, tid);
    store_rows<D, KB, NTH>(r, sV, tid);
  }
  const int nsteps = kv_steps<CAUSAL>(kb, KB, s), nch = (nsteps + C - 1) / C;
  // this chunk's query blocks of 32 (the walk starts at the diagonal)
  const int qstart = (CAUSAL ? k0 : 0) + 32 * C * chunk;
  const int nq = min(C, nsteps - C * chunk);
  struct Tile {
    u32x4 q[QP], o[QP];
    float l, d;
  };
  Tile t0, t1;
  auto fetch = [&](Tile& t, int q0) __attribute__((always_inline)) {
    load_rows<D, 32, NTH>(t.q, Qg, ld, q0, s, tid);
    load_rows<D, 32, NTH>(t.o, dOg, ldo, q0, s, tid);
    if (tid < 32) t.l = (q0 + tid < s) ? lseg[q0 + tid] * kLog2e : __builtin_inff();
    else if (tid < 64) t.d = (q0 + tid - 32 < s) ? Dg[q0 + tid - 32] : 0.f;
  };
  auto put = [&](const Tile& t, int buf) __attribute__((always_inline)) {
    store_rows<D, 32, NTH>(t.q, sQ[buf], tid);
    store_rows<D, 32, NTH>(t.o, sdO[buf], tid);
    if (tid < 32) sL[buf][tid] = t.l;
    else if (tid < 64) sDv[buf][tid - 32] = t.d;
  };
  if (nq > 0) fetch(t0, qstart);
  if (nq > 1) fetch(t1, qstart + 32);
  if (nq > 0) put(t0, 0);
  __syncthreads();

  f32x16 dk[DT], dv[DT];
#pragma unroll
  for (int i = 0; i < DT; ++i)
#pragma unroll
    for (int e = 0; e < 16; ++e) dk[i][e] = dv[i][e] = 0.f;
  // This wave's 32 keys as the other operand of S and dP, for the whole walk.
  bf16x8 kfr[KS], vfr[KS];
#pragma unroll
  for (int kk = 0; kk < KS; ++kk) {
    kfr[kk] = frag_rows<D>(sK, 32 * wave, kk, lane);
    vfr[kk] = frag_rows<D>(sV, 32 * wave, kk, lane);
  }

  // cur holds query block j+1 (stored to LDS at the end of the step); nxt is
  // free and receives block j+2.
  auto step = [&](int j, Tile& cur, Tile& nxt) __attribute__((always_inline)) {
    const int q0 = qstart + 32 * j, buf = j & 1;
    if (j + 2 < nq) fetch(nxt, q0 + 64);
    if (!(CAUSAL && kw > q0 + 31)) {
      const uint16_t* tq = sQ[buf];
      const uint16_t* td = sdO[buf];
      f32x16 S, dP;
#pragma unroll
      for (int e = 0; e < 16; ++e) S[e] = dP[e] = 0.f;
#pragma unroll
      for (int kk = 0; kk < KS; ++kk) {
        S = __builtin_amdgcn_mfma_f32_32x32x16_bf16(frag_rows<D>(tq, 0, kk, lane), kfr[kk], S, 0, 0, 0);
        dP = __builtin_amdgcn_mfma_f32_32x32x16_bf16(frag_rows<D>(td, 0, kk, lane), vfr[kk], dP, 0, 0, 0);
      }
      const int key = kw + lr;
      float p[16], ds[16];
      // P and dS. Causal: the mask is evaluated only where it can apply, when some
      // key of the wave's 32 lies above a query of the block or past the sequence end
      auto softmax = [&](auto masked) __attribute__((always_inline)) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const float4 L = *reinterpret_cast<const float4*>(&sL[buf][8 * g + 4 * hh]);
          const float4 Dd = *reinterpret_cast<const float4*>(&sDv[buf][8 * g + 4 * hh]);
          const float Lv[4] = {L.x, L.y, L.z, L.w}, Dq[4] = {Dd.x, Dd.y, Dd.z, Dd.w};
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            const int e = 4 * g + c, q = q0 + 8 * g + 4 * hh + c;
            float pv = __builtin_amdgcn_exp2f(__builtin_fmaf(S[e], scale_log2, -Lv[c]));
            if constexpr (decltype(masked)::value)
              if ((CAUSAL && key > q) || key >= s) pv = 0.f;
            p[e] = pv;
            ds[e] = pv * (dP[e] - Dq[c]);
          }
        }
      };
      if (!CAUSAL || kw + 31 > q0 || kw + 31 >= s)  // full attention keeps one path
        softmax(std::true_type{});
      else
        softmax(std::false_type{});
      const bf16x8 pa[2] = {pack8(p), pack8(p + 8)};
      const bf16x8 sa[2] = {pack8(ds), pack8(ds + 8)};
      const bf16x8 pl[2] = {pack8_lo(p, pa[0]), pack8_lo(p + 8, pa[1])};
      const bf16x8 sl[2] = {pack8_lo(ds, sa[0]), pack8_lo(ds + 8, sa[1])};
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int i = 0; i < DT; ++i) {
          const bf16x8 fo = frag_tr<D>(td, 16 * t, 32 * i, lane);
          const bf16x8 fq = frag_tr<D>(tq, 16 * t, 32 * i, lane);
          dv[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pa[t], fo, dv[i], 0, 0, 0);
          dk[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(sa[t], fq, dk[i], 0, 0, 0);
          dv[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pl[t], fo, dv[i], 0, 0, 0);
          dk[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(sl[t], fq, dk[i], 0, 0, 0);
        }
    }
    if (j + 1 < nq) put(cur, buf ^ 1);
    __syncthreads();
  };
  for (int j = 0; j < nq; j += 2) {
    step(j, t1, t0);
    if (j + 1 < nq) step(j + 1, t0, t1);
  }

  // accumulator lane: d column 32i + lr; register e: key kw + 8(e/4) + 4hh + e%4
  if (nch > 1) {
    const int64_t slot = ((int64_t)bh * nkb + kb) * kMaxChunks + chunk;
    float* pk = partK + slot * KB * D;
    float* pv = partV + slot * KB * D;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int kr = 32 * wave + 8 * (e >> 2) + 4 * hh + (e & 3);
#pragma unroll
      for (int i = 0; i < DT; ++i) {
        pk[kr * D + 32 * i + lr] = dk[i][e];
        pv[kr * D + 32 * i + lr] = dv[i][e];
      }
    }
    return;
  }
  uint16_t* dKg = dqkv + (int64_t)bi * s * ld + (int64_t)(Hl + head) * D;
  uint16_t* dVg = dqkv + (int64_t)bi * s * ld + (int64_t)(2 * Hl + head) * D;
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    const int key = kw + 8 * (e >> 2) + 4 * hh + (e & 3);
    if (key < s) {
#pragma unroll
      for (int i = 0; i < DT; ++i) {
        dKg[(int64_t)key * ld + 32 * i + lr] = (uint16_t)f32_to_bf16_bits(dk[i][e] * scale);
        dVg[(int64_t)key * ld + 32 * i + lr] = (uint16_t)f32_to_bf16_bits(dv[i][e]);
      }
    }
  }
}

// ------------------------------------------------------------------ dQ
template <int D, bool CAUSAL, int NW>
__device__ __forceinline__ void dq_item(int item, const uint16_t* __restrict__ qkv, const uint16_t* __restrict__ dO,
                                                     const float* __restrict__ lse, const float* __restrict__ Dv,
                                                     uint16_t* __restrict__ dqkv, float* __restrict__ partQ, int s,
                                                     int Hl, int BH, int nqb, int C, float scale_log2, float scale) {
  constexpr int NTH = NW * 64, QB = 32 * NW, KS = D / 16, DT = D / 32;
  constexpr int KP = 32 * D / 8 / NTH;
  __shared__ __attribute__((aligned(16))) uint16_t sK[2][32 * D];
  __shared__ __attribute__((aligned(16))) uint16_t sV[2][32 * D];

  const int bh = item % BH;
  int qb, chunk;
  chunk_of<CAUSAL, true>(item / BH, nqb, QB, s, C, qb, chunk);
  if (qb < 0) return;
  const int bi = bh / Hl, head = bh % Hl;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, lr = lane & 31, hh = lane >> 5;
  const int64_t ld = 3LL * Hl * D, ldo = (int64_t)Hl * D;
  const uint16_t* Qg = qkv + (int64_t)bi * s * ld + (int64_t)head * D;
  const uint16_t* Kg = Qg + (int64_t)Hl * D;
  const uint16_t* Vg = Qg + 2LL * Hl * D;
  const uint16_t* dOg = dO + (int64_t)bi * s * ldo + (int64_t)head * D;
  const int q0 = qb * QB, qw = q0 + 32 * wave, qrow = qw + lr;

  // This lane's query: its Q and dO columns as k-operand fragments over d.
  bf16x8 qf[KS], of[KS];
#pragma unroll
  for (int kk = 0; kk < KS; ++kk) {
    const int c = 16 * kk + 8 * hh;
    const bool ok = qrow < s;
    qf[kk] = ok ? *reinterpret_cast<const bf16x8*>(Qg + (int64_t)qrow * ld + c) : bf16x8{};
    of[kk] = ok ? *reinterpret_cast<const bf16x8*>(dOg + (int64_t)qrow * ldo + c) : bf16x8{};
  }
  const float Lq = qrow < s ? lse[(int64_t)bh * s + qrow] * kLog2e : __builtin_inff();
  const float Dq = qrow < s ? Dv[(int64_t)bh * s + qrow] : 0.f;

  const int nsteps = q_steps<CAUSAL>(qb, QB, s), nch = (nsteps + C - 1) / C;
  const int kbase = 32 * C * chunk;          // this chunk's first key
  const int nk = min(C, nsteps - C * chunk);  // its key blocks of 32
  u32x4 rk0[KP], rv0[KP], rk1[KP], rv1[KP];
  if (nk > 0) {
    load_rows<D, 32, NTH>(rk0, Kg, ld, kbase, s, tid);
    load_rows<D, 32, NTH>(rv0, Vg, ld, kbase, s, tid);
  }
  if (nk > 1) {
    load_rows<D, 32, NTH>(rk1, Kg, ld, kbase + 32, s, tid);
    load_rows<D, 32, NTH>(rv1, Vg, ld, kbase + 32, s, tid);
  }
  if (nk > 0) {
    store_rows<D, 32, NTH>(rk0, sK[0], tid);
    store_rows<D, 32, NTH>(rv0, sV[0], tid);
  }
  __syncthreads();

  f32x16 dq[DT];
#pragma unroll
  for (int i = 0; i < DT; ++i)
#pragma unroll
    for (int e = 0; e < 16; ++e) dq[i][e] = 0.f;

  // ck/cv hold key block j+1 (stored to LDS at the end of the step); fk/fv are
  // free and receive block j+2, two steps ahead of its use.
  auto step = [&](int j, u32x4 (&ck)[KP], u32x4 (&cv)[KP], u32x4 (&fk)[KP], u32x4 (&fv)[KP])
      __attribute__((always_inline)) {
    const int k0 = kbase + 32 * j, buf = j & 1;
    if (j + 2 < nk) {
      load_rows<D, 32, NTH>(fk, Kg, ld, k0 + 64, s, tid);
      load_rows<D, 32, NTH>(fv, Vg, ld, k0 + 64, s, tid);
    }
    if (!(CAUSAL && k0 > qw + 31)) {
      const uint16_t* tk = sK[buf];
      const uint16_t* tv = sV[buf];
      f32x16 S, dP;
#pragma unroll
      for (int e = 0; e < 16; ++e) S[e] = dP[e] = 0.f;
#pragma unroll
      for (int kk = 0; kk < KS; ++kk) {
        S = __builtin_amdgcn_mfma_f32_32x32x16_bf16(frag_rows<D>(tk, 0, kk, lane), qf[kk], S, 0, 0, 0);
        dP = __builtin_amdgcn_mfma_f32_32x32x16_bf16(frag_rows<D>(tv, 0, kk, lane), of[kk], dP, 0, 0, 0);
      }
      float ds[16];
      // causal: the mask only where some key of the 32 lies above a query of the wave or past the end
      auto softmax = [&](auto masked) __attribute__((always_inline)) {
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int key = k0 + 8 * (e >> 2) + 4 * hh + (e & 3);
          float pv = __builtin_amdgcn_exp2f(__builtin_fmaf(S[e], scale_log2, -Lq));
          if constexpr (decltype(masked)::value)
            if ((CAUSAL && key > qrow) || key >= s) pv = 0.f;
          ds[e] = pv * (dP[e] - Dq);
        }
      };
      if (!CAUSAL || k0 + 31 > qw || k0 + 31 >= s)  // full attention keeps one path
        softmax(std::true_type{});
      else
        softmax(std::false_type{});
      const bf16x8 sa[2] = {pack8(ds), pack8(ds + 8)};
      const bf16x8 sl[2] = {pack8_lo(ds, sa[0]), pack8_lo(ds + 8, sa[1])};
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int i = 0; i < DT; ++i) {
          const bf16x8 fk = frag_tr<D>(tk, 16 * t, 32 * i, lane);
          dq[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fk, sa[t], dq[i], 0, 0, 0);
          dq[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fk, sl[t], dq[i], 0, 0, 0);
        }
    }
    if (j + 1 < nk) {
      store_rows<D, 32, NTH>(ck, sK[buf ^ 1], tid);
      store_rows<D, 32, NTH>(cv, sV[buf ^ 1], tid);
    }
    __syncthreads();
  };
  for (int j = 0; j < nk; j += 2) {
    step(j, rk1, rv1, rk0, rv0);
    if (j + 1 < nk) step(j + 1, rk0, rv0, rk1, rv1);
  }

  // dQ^T accumulator lane: query column qrow; register e of tile i: d = 32i + 8(e/4) + 4hh + e%4
  if (nch > 1) {
    if (qrow < s) {
      float* pq = partQ + ((((int64_t)bh * nqb + qb) * kMaxChunks + chunk) * QB + (qrow - q0)) * D;
#pragma unroll
      for (int i = 0; i < DT; ++i)
#pragma unroll
        for (int g = 0; g < 4; ++g)
          *reinterpret_cast<f32x4*>(pq + 32 * i + 8 * g + 4 * hh) =
              f32x4{dq[i][4 * g], dq[i][4 * g + 1], dq[i][4 * g + 2], dq[i][4 * g + 3]};
    }
    return;
  }
  if (qrow < s) {
    uint16_t* dQg = dqkv + ((int64_t)bi * s + qrow) * ld + (int64_t)head * D;
#pragma unroll
    for (int i = 0; i < DT; ++i)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        uint2 u;
        u.x = pack_bf16x2(dq[i][4 * g] * scale, dq[i][4 * g + 1] * scale);
        u.y = pack_bf16x2(dq[i][4 * g + 2] * scale, dq[i][4 * g + 3] * scale);
        *reinterpret_cast<uint2*>(dQg + 32 * i + 8 * g + 4 * hh) = u;
      }
  }
}

// The dK/dV walks (items 0 .. nk_items - 1) and the dQ walks (the rest) in one
// grid: the two are independent, so the dQ items start on the CUs that the dK/dV
// items' tail leaves free instead of after the whole first grid has drained.
template <int D, bool CAUSAL, int NW>
__global__ __launch_bounds__(NW * 64) void dkdv_dq_kernel(const uint16_t* __restrict__ qkv,
                                                          const uint16_t* __restrict__ dO,
                                                          const float* __restrict__ lse,
                                                          const float* __restrict__ Dv, uint16_t* __restrict__ dqkv,
                                                          float* __restrict__ partQ, float* __restrict__ partK,
                                                          float* __restrict__ partV, int s, int Hl, int BH, int nblk,
                                                          int C, int nk_items, float scale_log2, float scale) {
  const int item = (int)blockIdx.x;
  if (item < nk_items)
    dkdv_item<D, CAUSAL, NW>(item, qkv, dO, lse, Dv, dqkv, partK, partV, s, Hl, BH, nblk, C, scale_log2, scale);
  else
    dq_item<D, CAUSAL, NW>(item - nk_items, qkv, dO, lse, Dv, dqkv, partQ, s, Hl, BH, nblk, C, scale_log2, scale);
}

// Workspace: D = rowsum(dO * O) [b*Hl*s], then the partial slots of dQ, dK, dV.
struct BwdLayout {
  int64_t d_bytes, q_bytes, kv_bytes;
  int nqb, nkb, C;
};
constexpr int kNW = 4;  // waves per workgroup (32 rows each) in both walks

inline int64_t r256(int64_t x) { return (x + 255) & ~int64_t(255); }

inline BwdLayout bwd_layout(int b, int s, int Hl, int d) {
  BwdLayout L;
  const int64_t BH = (int64_t)b * Hl;
  L.nqb = (s + 32 * kNW - 1) / (32 * kNW);
  L.nkb = L.nqb;
  const int max_steps = (s + 31) / 32;
  L.C = max(16, (max_steps + kMaxChunks - 1) / kMaxChunks);
  L.d_bytes = r256(BH * s * 4);
  const int64_t slots = L.C >= max_steps ? 0 : BH * L.nqb * kMaxChunks;  // no block splits when C covers every walk
  L.q_bytes = r256(slots * 32 * kNW * d * 4);
  L.kv_bytes = r256(slots * 32 * kNW * d * 4);
  return L;
}

template <int D, bool CAUSAL>
hipError_t launch_bwd(const uint16_t* qkv, const uint16_t* O, const uint16_t* dO, const float* lse, uint16_t* dqkv,
                      void* ws, int b, int s, int Hl, hipStream_t st) {
  const int64_t rows = (int64_t)b * s * Hl;
  if (rows == 0) return hipSuccess;
  const BwdLayout L = bwd_layout(b, s, Hl, D);
  char* w = static_cast<char*>(ws);
  float* Dws = reinterpret_cast<float*>(w);
  float* partQ = reinterpret_cast<float*>(w + L.d_bytes);
  float* partK = reinterpret_cast<float*>(w + L.d_bytes + L.q_bytes);
  float* partV = reinterpret_cast<float*>(w + L.d_bytes + L.q_bytes + L.kv_bytes);
  const int BH = b * Hl, R = 32 * kNW;
  int items_q = 0, items_k = 0, max_nc = 1;
  for (int i = 0; i < L.nqb; ++i) {
    const int nq = (q_steps<CAUSAL>(i, R, s) + L.C - 1) / L.C, nk = (kv_steps<CAUSAL>(i, R, s) + L.C - 1) / L.C;
    items_q += nq;
    items_k += nk;
    max_nc = max(max_nc, max(nq, nk));
  }
  if (max_nc > 1 && L.q_bytes == 0) return hipErrorInvalidValue;
  if ((int64_t)BH * (items_q + items_k) > 0x7fffffffLL) return hipErrorInvalidValue;  // grid.x range
  const float scale = 1.f / sqrtf((float)D), scale_log2 = kLog2e * scale;
  hipLaunchKernelGGL(rowdot_kernel, dim3((unsigned)((rows + 15) / 16)), dim3(256), 0, st, dO, O, Dws, s, Hl, D, rows);
  hipLaunchKernelGGL((dkdv_dq_kernel<D, CAUSAL, kNW>), dim3((unsigned)((int64_t)BH * (items_k + items_q))),
                     dim3(kNW * 64), 0, st, qkv, dO, lse, Dws, dqkv, partQ, partK, partV, s, Hl, BH, L.nqb, L.C,
                     BH * items_k, scale_log2, scale);
  if (max_nc > 1) {
    const dim3 grid((unsigned)((int64_t)BH * L.nqb), (unsigned)((R * D / 4 + 255) / 256), 3);
    hipLaunchKernelGGL((combine_kernel<D, CAUSAL>), grid, dim3(256), 0, st, partQ, partK, partV, dqkv, s, Hl, L.nqb,
                       R, L.C, scale);
  }
  return hipGetLastError();
}

// ------------------------------------------------------------------ wide heads
// Heads of d = 384 walk the same way, but one wave cannot hold the K and V
// fragments of 32 keys over all 384 d (192 registers per lane) next to 384-wide
// dK and dV accumulators. A workgroup of four waves takes a block of 64 keys
// (dK/dV walk) or 64 queries (dQ walk), two halves of 32, and each step's work
// splits two ways:
//   * scores: wave h (h = 0, 1) forms S for half h over all d from fragments it
//     holds for the whole walk (K for the dK/dV walk, Q for the dQ walk), wave
//     2 + h forms dP for half h (from V, or dO); the S wave turns S into P and
//     hands it through LDS to the dP wave of its half, which forms dS; both
//     leave their bf16 hi/lo operand fragments in LDS;
//   * products: wave w accumulates the d columns [96w, 96w + 96) of the
//     gradients of both halves from those fragments and the staged tile.
// Three barriers a step: P ready, dS ready, next tile staged. For a half whose
// keys all lie above the step's queries (or past the end) the score waves skip
// their MFMAs and hand on zero fragments; the products run for both halves
// regardless (per-half branches there split the MFMA stream into small blocks).
// Walks are cut into chunks as above, and combine_kernel adds the chunks'
// partials.
constexpr int kWideD = 384;
constexpr int kWideTileB = 32 * kWideD * 2;             // bytes of a [32][384] bf16 tile
constexpr int kWideOffB = 2 * kWideTileB;               // second pair of tiles (dO or V)
constexpr int kWideOffXP = 4 * kWideTileB;              // P, float32 [half][4][lane] x4
constexpr int kWideOffXPb = kWideOffXP + 2 * 4 * 64 * 16;   // P hi/lo fragments [half][4][lane]
constexpr int kWideOffXSb = kWideOffXPb + 2 * 4 * 64 * 16;  // dS hi/lo fragments [half][4][lane]
constexpr int kWideOffL = kWideOffXSb + 2 * 4 * 64 * 16;    // lse (log2 units) and D [2][64]
constexpr int kWideLds = kWideOffL + 2 * 64 * 4;            // 123392 bytes

// Block rows are 64 (two halves of 32) in both wide walks.
constexpr int kWideR = 64;

typedef int i32x4 __attribute__((ext_vector_type(4)));
constexpr uint32_t kDmaOOB = 0x7ffffff0u;  // buffer offset past every range: reads as zero

__device__ __forceinline__ uint32_t lds_u32(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// Rows [r0, r0 + 32) of one head's 384 columns of a [rows][ld] bf16 tensor,
// straight from memory into a swizzled [32][384] LDS tile with
// buffer_load_dwordx4 ... lds (rows at or past `rows` read as zero). Wave w of
// four issues 6 of the tile's 24 1-KB pieces; physical chunk P of the tile (row
// P / 48, position P % 48) receives logical chunk (P % 48) ^ swz384(row). The loads
// complete asynchronously: s_waitcnt vmcnt(0) before the barrier that publishes
// the tile. Issued as inline asm (no register outputs), so the compiler does
// not wait for them before unrelated LDS reads.
__device__ __forceinline__ void dma_tile384(const uint16_t* g, int64_t ld, int r0, int rows, uint16_t* tile,
                                            int wave, int lane) {
  const uint64_t a = reinterpret_cast<uint64_t>(g + (int64_t)r0 * ld);
  const i32x4 rs = {(int)(uint32_t)a, (int)((a >> 32) & 0xffff), (int)(uint32_t)(32 * ld * 2), 0x00020000};
  const uint32_t base = lds_u32(tile);
#pragma unroll
  for (int o = 0; o < 6; ++o) {
    const int P = (wave * 6 + o) * 64 + lane, r = P / 48, c = (P % 48) ^ swz384(r);
    const uint32_t off = (r0 + r < rows) ? (uint32_t)(r * ld * 2 + c * 16) : kDmaOOB;
    const uint32_t dst = __builtin_amdgcn_readfirstlane(base + (uint32_t)((wave * 6 + o) * 1024));
    asm volatile("buffer_load_dwordx4 %0, %1, 0 offen lds" ::"v"(off), "s"(rs), "{m0}"(dst) : "memory");
  }
}

// A score tile over all 384 d: 24 MFMAs from the staged tile t (row operand)
// and the fragments fr held for the walk (column operand), with the tile's
// fragment reads issued four ahead of the MFMAs that use them.
__device__ __forceinline__ f32x16 score384(const uint16_t* t, const bf16x8 (&fr)[kWideD / 16], int lane) {
  constexpr int KS = kWideD / 16, AHEAD = 4;
  f32x16 acc;
#pragma unroll
  for (int e = 0; e < 16; ++e) acc[e] = 0.f;
  bf16x8 a[KS];
#pragma unroll
  for (int kk = 0; kk < AHEAD; ++kk) a[kk] = frag_rows<kWideD>(t, 0, kk, lane);
#pragma unroll
  for (int kk = 0; kk < KS; ++kk) {
    if (kk + AHEAD < KS) a[kk + AHEAD] = frag_rows<kWideD>(t, 0, kk + AHEAD, lane);
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[kk], fr[kk], acc, 0, 0, 0);
  }
  __builtin_amdgcn_sched_group_barrier(0x100, AHEAD, 0);  // DS reads
#pragma unroll
  for (int kk = 0; kk < KS - AHEAD; ++kk) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // DS read
  }
  __builtin_amdgcn_sched_group_barrier(0x008, AHEAD, 0);
  return acc;
}

template <bool CAUSAL>
__device__ __forceinline__ void dkdv_wide_item(int item, char* lds, const uint16_t* __restrict__ qkv,
                                               const uint16_t* __restrict__ dO, const float* __restrict__ lse,
                                               const float* __restrict__ Dv, uint16_t* __restrict__ dqkv,
                                               float* __restrict__ partK, float* __restrict__ partV, int s, int Hl,
                                               int BH, int nkb, int C, float scale_log2, float scale) {
  constexpr int D = kWideD, KS = D / 16;
  uint16_t* const sQ0 = reinterpret_cast<uint16_t*>(lds);
  uint16_t* const sdO0 = reinterpret_cast<uint16_t*>(lds + kWideOffB);
  f32x4* const xP = reinterpret_cast<f32x4*>(lds + kWideOffXP);
  u32x4* const xPb = reinterpret_cast<u32x4*>(lds + kWideOffXPb);
  u32x4* const xSb = reinterpret_cast<u32x4*>(lds + kWideOffXSb);
  float* const sLD = reinterpret_cast<float*>(lds + kWideOffL);  // [buf][lse (log2 units) x 32 | D x 32]

  const int bh = item % BH;
  int kb, chunk;
  chunk_of<CAUSAL, false>(item / BH, nkb, kWideR, s, C, kb, chunk);
  if (kb < 0) return;
  const int bi = bh / Hl, head = bh % Hl;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, lr = lane & 31, hh = lane >> 5;
  const int half = wave & 1;
  const bool sw = wave < 2;  // S wave; else dP wave
  const int64_t ld = 3LL * Hl * D, ldo = (int64_t)Hl * D;
  const uint16_t* Qg = qkv + (int64_t)bi * s * ld + (int64_t)head * D;
  const uint16_t* Kg = Qg + (int64_t)Hl * D;
  const uint16_t* Vg = Qg + 2LL * Hl * D;
  const uint16_t* dOg = dO + (int64_t)bi * s * ldo + (int64_t)head * D;
  const float* lseg = lse + (int64_t)bh * s;
  const float* Dg = Dv + (int64_t)bh * s;
  const int k0 = kb * kWideR, kh = k0 + 32 * half;

  // K (S wave) or V (dP wave) of key kh + lr over all d: the score product's column operand
  bf16x8 fr[KS];
  {
    const bool ok = kh + lr < s;
    const uint16_t* src = (sw ? Kg : Vg) + (int64_t)(ok ? kh + lr : 0) * ld + 8 * hh;
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) fr[kk] = ok ? *reinterpret_cast<const bf16x8*>(src + 16 * kk) : bf16x8{};
    // consume the loads here: a first use inside the walk would make the compiler
    // wait there on every step, and so for the tile DMAs still in flight
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) asm volatile("" : "+v"(fr[kk]));
  }

  const int nsteps = kv_steps<CAUSAL>(kb, kWideR, s), nch = (nsteps + C - 1) / C;
  const int qstart = (CAUSAL ? k0 : 0) + 32 * C * chunk;
  const int nq = min(C, nsteps - C * chunk);
  // the next query block: Q and dO tiles by DMA into LDS buffer buf, lse and D through registers
  // (thread t < 32 loads the lse of query q0 + t, thread 32 + t its D; the value is
  // first used at put, after the tiles' own wait)
  float rx = 0.f;
  auto fetch = [&](int q0, int buf) __attribute__((always_inline)) {
    const int q = q0 + (tid & 31);
    if (tid < 64) rx = q < s ? (tid < 32 ? lseg[q] : Dg[q]) : (tid < 32 ? __builtin_inff() : 0.f);
    dma_tile384(Qg, ld, q0, s, sQ0 + buf * 32 * D, wave, lane);
    dma_tile384(dOg, ldo, q0, s, sdO0 + buf * 32 * D, wave, lane);
  };
  auto put = [&](int buf) __attribute__((always_inline)) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    if (tid < 64) sLD[buf * 64 + tid] = tid < 32 ? rx * kLog2e : rx;
  };
  fetch(qstart, 0);
  put(0);
  __syncthreads();

  f32x16 dk[2][3], dv[2][3];
#pragma unroll
  for (int hv = 0; hv < 2; ++hv)
#pragma unroll
    for (int i = 0; i < 3; ++i)
#pragma unroll
      for (int e = 0; e < 16; ++e) dk[hv][i][e] = dv[hv][i][e] = 0.f;

  for (int j = 0; j < nq; ++j) {
    const int q0 = qstart + 32 * j, buf = j & 1;
    if (j + 1 < nq) fetch(q0 + 32, buf ^ 1);
    const uint16_t* tq = sQ0 + buf * 32 * D;
    const uint16_t* td = sdO0 + buf * 32 * D;
    // half hv takes part unless all its keys lie above every query of the block or past the end
    const bool mine = kh < s && !(CAUSAL && kh > q0 + 31);

    // scores: S = Q K^T (S waves) or dP = dO V^T (dP waves) for this half;
    // lane: key kh + lr, register e: query q0 + 8(e/4) + 4hh + e%4
    f32x16 acc;
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[e] = 0.f;
    if (mine) acc = score384(sw ? tq : td, fr, lane);
    if (sw) {
      const int key = kh + lr;
      float p[16];
      auto softmax = [&](auto masked) __attribute__((always_inline)) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const float4 L = *reinterpret_cast<const float4*>(&sLD[buf * 64 + 8 * g + 4 * hh]);
          const float Lv[4] = {L.x, L.y, L.z, L.w};
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            const int e = 4 * g + c, q = q0 + 8 * g + 4 * hh + c;
            float pv = __builtin_amdgcn_exp2f(__builtin_fmaf(acc[e], scale_log2, -Lv[c]));
            if constexpr (decltype(masked)::value)
              if ((CAUSAL && key > q) || key >= s) pv = 0.f;
            p[e] = pv;
          }
        }
      };
      if (!mine) {  // a dead half hands on zeros
#pragma unroll
        for (int e = 0; e < 16; ++e) p[e] = 0.f;
      } else if (!CAUSAL || kh + 31 > q0 || kh + 31 >= s) {
        softmax(std::true_type{});
      } else {
        softmax(std::false_type{});
      }
#pragma unroll
      for (int g = 0; g < 4; ++g) xP[(half * 4 + g) * 64 + lane] = f32x4{p[4 * g], p[4 * g + 1], p[4 * g + 2], p[4 * g + 3]};
      const bf16x8 a0 = pack8(p), a1 = pack8(p + 8);
      xPb[(half * 4 + 0) * 64 + lane] = __builtin_bit_cast(u32x4, a0);
      xPb[(half * 4 + 1) * 64 + lane] = __builtin_bit_cast(u32x4, a1);
      xPb[(half * 4 + 2) * 64 + lane] = __builtin_bit_cast(u32x4, pack8_lo(p, a0));
      xPb[(half * 4 + 3) * 64 + lane] = __builtin_bit_cast(u32x4, pack8_lo(p + 8, a1));
    }
    __syncthreads();
    if (!sw) {
      float ds[16];
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f32x4 pv = xP[(half * 4 + g) * 64 + lane];
        const float4 Dd = *reinterpret_cast<const float4*>(&sLD[buf * 64 + 32 + 8 * g + 4 * hh]);
        ds[4 * g + 0] = pv[0] * (acc[4 * g + 0] - Dd.x);
        ds[4 * g + 1] = pv[1] * (acc[4 * g + 1] - Dd.y);
        ds[4 * g + 2] = pv[2] * (acc[4 * g + 2] - Dd.z);
        ds[4 * g + 3] = pv[3] * (acc[4 * g + 3] - Dd.w);
      }
      const bf16x8 a0 = pack8(ds), a1 = pack8(ds + 8);
      xSb[(half * 4 + 0) * 64 + lane] = __builtin_bit_cast(u32x4, a0);
      xSb[(half * 4 + 1) * 64 + lane] = __builtin_bit_cast(u32x4, a1);
      xSb[(half * 4 + 2) * 64 + lane] = __builtin_bit_cast(u32x4, pack8_lo(ds, a0));
      xSb[(half * 4 + 3) * 64 + lane] = __builtin_bit_cast(u32x4, pack8_lo(ds + 8, a1));
    }
    __syncthreads();

    // dV += P^T dO and dK += dS^T Q over this wave's 96 d columns, both halves
    // (a dead half's fragments are zero), one 16-query k-slice t at a time (P and
    // dS fragments: hi, lo)
    auto products = [&]() __attribute__((always_inline)) {
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        bf16x8 ph[2], pl[2], sh[2], sl[2];
#pragma unroll
        for (int hv = 0; hv < 2; ++hv)
          {
            ph[hv] = __builtin_bit_cast(bf16x8, xPb[(hv * 4 + t) * 64 + lane]);
            pl[hv] = __builtin_bit_cast(bf16x8, xPb[(hv * 4 + 2 + t) * 64 + lane]);
            sh[hv] = __builtin_bit_cast(bf16x8, xSb[(hv * 4 + t) * 64 + lane]);
            sl[hv] = __builtin_bit_cast(bf16x8, xSb[(hv * 4 + 2 + t) * 64 + lane]);
          }
#pragma unroll
        for (int i = 0; i < 3; ++i) {
          const bf16x8 fo = frag_tr<D>(td, 16 * t, 96 * wave + 32 * i, lane);
          const bf16x8 fq = frag_tr<D>(tq, 16 * t, 96 * wave + 32 * i, lane);
#pragma unroll
          for (int hv = 0; hv < 2; ++hv)
            {
              dv[hv][i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ph[hv], fo, dv[hv][i], 0, 0, 0);
              dv[hv][i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pl[hv], fo, dv[hv][i], 0, 0, 0);
              dk[hv][i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(sh[hv], fq, dk[hv][i], 0, 0, 0);
              dk[hv][i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(sl[hv], fq, dk[hv][i], 0, 0, 0);
            }
        }
      }
    };
    products();
    if (j + 1 < nq) put(buf ^ 1);
    __syncthreads();
  }

  // accumulator lane: d column 96w + 32i + lr; register e: key k0 + 32hv + 8(e/4) + 4hh + e%4
  if (nch > 1) {
    const int64_t slot = ((int64_t)bh * nkb + kb) * kMaxChunks + chunk;
    float* pk = partK + slot * kWideR * D;
    float* pv = partV + slot * kWideR * D;
#pragma unroll
    for (int hv = 0; hv < 2; ++hv)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int kr = 32 * hv + 8 * (e >> 2) + 4 * hh + (e & 3);
#pragma unroll
        for (int i = 0; i < 3; ++i) {
          pk[kr * D + 96 * wave + 32 * i + lr] = dk[hv][i][e];
          pv[kr * D + 96 * wave + 32 * i + lr] = dv[hv][i][e];
        }
      }
    return;
  }
  uint16_t* dKg = dqkv + (int64_t)bi * s * ld + (int64_t)(Hl + head) * D;
  uint16_t* dVg = dqkv + (int64_t)bi * s * ld + (int64_t)(2 * Hl + head) * D;
#pragma unroll
  for (int hv = 0; hv < 2; ++hv)
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int key = k0 + 32 * hv + 8 * (e >> 2) + 4 * hh + (e & 3);
      if (key < s) {
#pragma unroll
        for (int i = 0; i < 3; ++i) {
          dKg[(int64_t)key * ld + 96 * wave + 32 * i + lr] = (uint16_t)f32_to_bf16_bits(dk[hv][i][e] * scale);
          dVg[(int64_t)key * ld + 96 * wave + 32 * i + lr] = (uint16_t)f32_to_bf16_bits(dv[hv][i][e]);
        }
      }
    }
}

template <bool CAUSAL>
__device__ __forceinline__ void dq_wide_item(int item, char* lds, const uint16_t* __restrict__ qkv,
                                             const uint16_t* __restrict__ dO, const float* __restrict__ lse,
                                             const float* __restrict__ Dv, uint16_t* __restrict__ dqkv,
                                             float* __restrict__ partQ, int s, int Hl, int BH, int nqb, int C,
                                             float scale_log2, float scale) {
  constexpr int D = kWideD, KS = D / 16;
  uint16_t* const sK0 = reinterpret_cast<uint16_t*>(lds);
  uint16_t* const sV0 = reinterpret_cast<uint16_t*>(lds + kWideOffB);
  f32x4* const xP = reinterpret_cast<f32x4*>(lds + kWideOffXP);
  u32x4* const xSb = reinterpret_cast<u32x4*>(lds + kWideOffXSb);

  const int bh = item % BH;
  int qb, chunk;
  chunk_of<CAUSAL, true>(item / BH, nqb, kWideR, s, C, qb, chunk);
  if (qb < 0) return;
  const int bi = bh / Hl, head = bh % Hl;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, lr = lane & 31, hh = lane >> 5;
  const int half = wave & 1;
  const bool sw = wave < 2;
  const int64_t ld = 3LL * Hl * D, ldo = (int64_t)Hl * D;
  const uint16_t* Qg = qkv + (int64_t)bi * s * ld + (int64_t)head * D;
  const uint16_t* Kg = Qg + (int64_t)Hl * D;
  const uint16_t* Vg = Qg + 2LL * Hl * D;
  const uint16_t* dOg = dO + (int64_t)bi * s * ldo + (int64_t)head * D;
  const int q0 = qb * kWideR, qh = q0 + 32 * half, qrow = qh + lr;

  // Q (S wave) or dO (dP wave) of query qrow over all d: the score product's column operand
  bf16x8 fr[KS];
  float Lq = __builtin_inff(), Dq = 0.f;
  {
    const bool ok = qrow < s;
    const uint16_t* src = (sw ? Qg + (int64_t)(ok ? qrow : 0) * ld : dOg + (int64_t)(ok ? qrow : 0) * ldo) + 8 * hh;
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) fr[kk] = ok ? *reinterpret_cast<const bf16x8*>(src + 16 * kk) : bf16x8{};
    if (ok) {
      if (sw) Lq = lse[(int64_t)bh * s + qrow] * kLog2e;
      else Dq = Dv[(int64_t)bh * s + qrow];
    }
    // consume the loads before the walk (see dkdv_wide_item)
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) asm volatile("" : "+v"(fr[kk]));
    asm volatile("" : "+v"(Lq), "+v"(Dq));
  }

  const int nsteps = q_steps<CAUSAL>(qb, kWideR, s), nch = (nsteps + C - 1) / C;
  const int kbase = 32 * C * chunk;
  const int nk = min(C, nsteps - C * chunk);
  // the next key block: K and V tiles by DMA into LDS buffer buf
  auto fetch = [&](int k0, int buf) __attribute__((always_inline)) {
    dma_tile384(Kg, ld, k0, s, sK0 + buf * 32 * D, wave, lane);
    dma_tile384(Vg, ld, k0, s, sV0 + buf * 32 * D, wave, lane);
  };
  auto put = [&]() __attribute__((always_inline)) { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); };
  fetch(kbase, 0);
  put();
  __syncthreads();

  f32x16 dq[2][3];
#pragma unroll
  for (int hv = 0; hv < 2; ++hv)
#pragma unroll
    for (int i = 0; i < 3; ++i)
#pragma unroll
      for (int e = 0; e < 16; ++e) dq[hv][i][e] = 0.f;

  for (int j = 0; j < nk; ++j) {
    const int k0 = kbase + 32 * j, buf = j & 1;
    if (j + 1 < nk) fetch(k0 + 32, buf ^ 1);
    const uint16_t* tk = sK0 + buf * 32 * D;
    const uint16_t* tv = sV0 + buf * 32 * D;
    // half hv takes part unless all its queries lie past the end or below every key of the block
    const bool mine = qh < s && !(CAUSAL && k0 > qh + 31);

    // scores, transposed: S^T = K Q^T (S waves) or dP^T = V dO^T (dP waves) for this half;
    // lane: query qrow, register e: key k0 + 8(e/4) + 4hh + e%4
    f32x16 acc;
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[e] = 0.f;
    if (mine) acc = score384(sw ? tk : tv, fr, lane);
    if (sw) {
      float p[16];
      auto softmax = [&](auto masked) __attribute__((always_inline)) {
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int key = k0 + 8 * (e >> 2) + 4 * hh + (e & 3);
          float pv = __builtin_amdgcn_exp2f(__builtin_fmaf(acc[e], scale_log2, -Lq));
          if constexpr (decltype(masked)::value)
            if ((CAUSAL && key > qrow) || key >= s) pv = 0.f;
          p[e] = pv;
        }
      };
      if (!mine) {  // a dead half hands on zeros
#pragma unroll
        for (int e = 0; e < 16; ++e) p[e] = 0.f;
      } else if (!CAUSAL || k0 + 31 > qh || k0 + 31 >= s) {
        softmax(std::true_type{});
      } else {
        softmax(std::false_type{});
      }
#pragma unroll
      for (int g = 0; g < 4; ++g) xP[(half * 4 + g) * 64 + lane] = f32x4{p[4 * g], p[4 * g + 1], p[4 * g + 2], p[4 * g + 3]};
    }
    __syncthreads();
    if (!sw) {
      float ds[16];
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f32x4 pv = xP[(half * 4 + g) * 64 + lane];
#pragma unroll
        for (int c = 0; c < 4; ++c) ds[4 * g + c] = pv[c] * (acc[4 * g + c] - Dq);
      }
      const bf16x8 a0 = pack8(ds), a1 = pack8(ds + 8);
      xSb[(half * 4 + 0) * 64 + lane] = __builtin_bit_cast(u32x4, a0);
      xSb[(half * 4 + 1) * 64 + lane] = __builtin_bit_cast(u32x4, a1);
      xSb[(half * 4 + 2) * 64 + lane] = __builtin_bit_cast(u32x4, pack8_lo(ds, a0));
      xSb[(half * 4 + 3) * 64 + lane] = __builtin_bit_cast(u32x4, pack8_lo(ds + 8, a1));
    }
    __syncthreads();

    // dQ^T += K^T dS^T over this wave's 96 d rows, both halves (a dead half's
    // fragments are zero), one 16-key k-slice t at a time
    auto products = [&]() __attribute__((always_inline)) {
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        bf16x8 sh[2], sl[2];
#pragma unroll
        for (int hv = 0; hv < 2; ++hv)
          {
            sh[hv] = __builtin_bit_cast(bf16x8, xSb[(hv * 4 + t) * 64 + lane]);
            sl[hv] = __builtin_bit_cast(bf16x8, xSb[(hv * 4 + 2 + t) * 64 + lane]);
          }
#pragma unroll
        for (int i = 0; i < 3; ++i) {
          const bf16x8 fk = frag_tr<D>(tk, 16 * t, 96 * wave + 32 * i, lane);
#pragma unroll
          for (int hv = 0; hv < 2; ++hv)
            {
              dq[hv][i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fk, sh[hv], dq[hv][i], 0, 0, 0);
              dq[hv][i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fk, sl[hv], dq[hv][i], 0, 0, 0);
            }
        }
      }
    };
    products();
    if (j + 1 < nk) put();
    __syncthreads();
  }

  // dQ^T accumulator lane: query q0 + 32hv + lr; register e of tile i: d = 96w + 32i + 8(e/4) + 4hh + e%4
  if (nch > 1) {
#pragma unroll
    for (int hv = 0; hv < 2; ++hv) {
      const int row = 32 * hv + lr;
      if (q0 + row >= s) continue;
      float* pq = partQ + ((((int64_t)bh * nqb + qb) * kMaxChunks + chunk) * kWideR + row) * D;
#pragma unroll
      for (int i = 0; i < 3; ++i)
#pragma unroll
        for (int g = 0; g < 4; ++g)
          *reinterpret_cast<f32x4*>(pq + 96 * wave + 32 * i + 8 * g + 4 * hh) =
              f32x4{dq[hv][i][4 * g], dq[hv][i][4 * g + 1], dq[hv][i][4 * g + 2], dq[hv][i][4 * g + 3]};
    }
    return;
  }
#pragma unroll
  for (int hv = 0; hv < 2; ++hv) {
    const int q = q0 + 32 * hv + lr;
    if (q >= s) continue;
    uint16_t* dQg = dqkv + ((int64_t)bi * s + q) * ld + (int64_t)head * D;
#pragma unroll
    for (int i = 0; i < 3; ++i)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        uint2 u;
        u.x = pack_bf16x2(dq[hv][i][4 * g] * scale, dq[hv][i][4 * g + 1] * scale);
        u.y = pack_bf16x2(dq[hv][i][4 * g + 2] * scale, dq[hv][i][4 * g + 3] * scale);
        *reinterpret_cast<uint2*>(dQg + 96 * wave + 32 * i + 8 * g + 4 * hh) = u;
      }
  }
}

// The wide dK/dV walks (items 0 .. nk_items - 1) and dQ walks in one grid; the
// two kinds share one LDS area.
template <bool CAUSAL>
__global__ __launch_bounds__(256) void dkdv_dq_wide_kernel(const uint16_t* __restrict__ qkv,
                                                           const uint16_t* __restrict__ dO,
                                                           const float* __restrict__ lse,
                                                           const float* __restrict__ Dv, uint16_t* __restrict__ dqkv,
                                                           float* __restrict__ partQ, float* __restrict__ partK,
                                                           float* __restrict__ partV, int s, int Hl, int BH, int nblk,
                                                           int C, int nk_items, float scale_log2, float scale) {
  __shared__ __attribute__((aligned(16))) char lds[kWideLds];
  const int item = (int)blockIdx.x;
  if (item < nk_items)
    dkdv_wide_item<CAUSAL>(item, lds, qkv, dO, lse, Dv, dqkv, partK, partV, s, Hl, BH, nblk, C, scale_log2, scale);
  else
    dq_wide_item<CAUSAL>(item - nk_items, lds, qkv, dO, lse, Dv, dqkv, partQ, s, Hl, BH, nblk, C, scale_log2,
                         scale);
}

inline BwdLayout bwd_layout_wide(int b, int s, int Hl) {
  BwdLayout L;
  const int64_t BH = (int64_t)b * Hl;
  L.nqb = (s + kWideR - 1) / kWideR;
  L.nkb = L.nqb;
  const int max_steps = (s + 31) / 32;
  L.C = max(16, (max_steps + kMaxChunks - 1) / kMaxChunks);
  L.d_bytes = r256(BH * s * 4);
  const int64_t slots = L.C >= max_steps ? 0 : BH * L.nqb * kMaxChunks;
  L.q_bytes = r256(slots * kWideR * kWideD * 4);
  L.kv_bytes = L.q_bytes;
  return L;
}

template <bool CAUSAL>
hipError_t launch_bwd_wide(const uint16_t* qkv, const uint16_t* O, const uint16_t* dO, const float* lse,
                           uint16_t* dqkv, void* ws, int b, int s, int Hl, hipStream_t st) {
  constexpr int D = kWideD;
  const int64_t rows = (int64_t)b * s * Hl;
  if (rows == 0) return hipSuccess;
  const BwdLayout L = bwd_layout_wide(b, s, Hl);
  char* w = static_cast<char*>(ws);
  float* Dws = reinterpret_cast<float*>(w);
  float* partQ = reinterpret_cast<float*>(w + L.d_bytes);
  float* partK = reinterpret_cast<float*>(w + L.d_bytes + L.q_bytes);
  float* partV = reinterpret_cast<float*>(w + L.d_bytes + L.q_bytes + L.kv_bytes);
  const int BH = b * Hl;
  int items_q = 0, items_k = 0, max_nc = 1;
  for (int i = 0; i < L.nqb; ++i) {
    const int nq = (q_steps<CAUSAL>(i, kWideR, s) + L.C - 1) / L.C;
    const int nk = (kv_steps<CAUSAL>(i, kWideR, s) + L.C - 1) / L.C;
    items_q += nq;
    items_k += nk;
    max_nc = max(max_nc, max(nq, nk));
  }
  if (max_nc > 1 && L.q_bytes == 0) return hipErrorInvalidValue;
  if ((int64_t)BH * (items_q + items_k) > 0x7fffffffLL) return hipErrorInvalidValue;
  const float scale = 1.f / sqrtf((float)D), scale_log2 = kLog2e * scale;
  hipLaunchKernelGGL(rowdot_kernel, dim3((unsigned)((rows + 15) / 16)), dim3(256), 0, st, dO, O, Dws, s, Hl, D, rows);
  hipLaunchKernelGGL((dkdv_dq_wide_kernel<CAUSAL>), dim3((unsigned)((int64_t)BH * (items_k + items_q))), dim3(256),
                     0, st, qkv, dO, lse, Dws, dqkv, partQ, partK, partV, s, Hl, BH, L.nqb, L.C, BH * items_k,
                     scale_log2, scale);
  if (max_nc > 1) {
    const dim3 grid((unsigned)((int64_t)BH * L.nqb), (unsigned)((kWideR * D / 4 + 255) / 256), 3);
    hipLaunchKernelGGL((combine_kernel<D, CAUSAL>), grid, dim3(256), 0, st, partQ, partK, partV, dqkv, s, Hl, L.nqb,
                       kWideR, L.C, scale);
  }
  return hipGetLastError();
}

}  // namespace

size_t attn_bwd_workspace(int b, int s, int Hl, int d) {
  if (b <= 0 || s <= 0 || Hl <= 0) return 0;
  if (d == kWideD) {
    const BwdLayout L = bwd_layout_wide(b, s, Hl);
    return (size_t)(L.d_bytes + L.q_bytes + 2 * L.kv_bytes);
  }
  const BwdLayout L = bwd_layout(b, s, Hl, d);
  return (size_t)(L.d_bytes + L.q_bytes + 2 * L.kv_bytes);
}

hipError_t attn_bwd(const uint16_t* qkv, const uint16_t* O, const uint16_t* dO, const float* lse, uint16_t* dqkv,
                    void* ws, int b, int s, int Hl, int d, bool causal, hipStream_t st) {
  if (d == 128)
    return causal ? launch_bwd<128, true>(qkv, O, dO, lse, dqkv, ws, b, s, Hl, st)
                  : launch_bwd<128, false>(qkv, O, dO, lse, dqkv, ws, b, s, Hl, st);
  if (d == 64)
    return causal ? launch_bwd<64, true>(qkv, O, dO, lse, dqkv, ws, b, s, Hl, st)
                  : launch_bwd<64, false>(qkv, O, dO, lse, dqkv, ws, b, s, Hl, st);
  if (d == kWideD)
    return causal ? launch_bwd_wide<true>(qkv, O, dO, lse, dqkv, ws, b, s, Hl, st)
                  : launch_bwd_wide<false>(qkv, O, dO, lse, dqkv, ws, b, s, Hl, st);
  return hipErrorInvalidValue;
}

}  // namespace tps
