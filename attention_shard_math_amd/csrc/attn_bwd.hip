// Backward of the fused causal attention (gfx950), deterministic, no atomics.
//
// With P = exp(S/sqrt(d) - lse) recomputed from the forward's log-sum-exp:
//   dV = P^T dO,  dP = dO V^T,  dS = P * (dP - D),  D = rowsum(dO * O),
//   dQ = dS K / sqrt(d),  dK = dS^T Q / sqrt(d).
// Three launches:
//   * attn_bwd_rowdot — D per (query, head), 16 lanes per row of 128;
//   * attn_bwd_dkdv   — one workgroup per (sequence, head, block of 32*NW keys),
//     wave w owning 32 keys (their K and V fragments, dK and dV in registers);
//     it walks the query blocks of 32 that can see its keys, with each block's Q
//     and dO staged in LDS (double-buffered) and shared by the waves;
//   * attn_bwd_dq     — one workgroup per (sequence, head, block of 32*NW
//     queries), wave w owning 32 queries whose Q and dO fragments sit in
//     registers; it walks the key blocks of 32 up to the diagonal, K and V
//     staged in LDS.
// The staged tiles are loaded into registers two steps ahead of their use (two
// register sets, the loop unrolled by two), so a step's compute covers the
// global-load latency of the tile after next.
// Both big kernels run their products on v_mfma_f32_32x32x16_bf16. The score
// tile comes out of the MFMA with a lane owning one column and 16 rows
// {8(e/4) + 4(l/32) + e%4}; those 16 values (8 per 16-row k-slice, packed to
// bf16) are used directly as the k-operand of the next product, taking the
// k-slice in that permuted order. The other operand of that product is read
// from LDS with ds_read_b64_tr_b16, whose 4-row groups are picked to match
// the same order, so no score tile goes through LDS.
//
// LDS rows are 256 bytes (128 bf16); 16-byte chunk c of row r is stored at
// c ^ swz(r), swz(r) = ((r & 7) << 1) | ((r >> 3) & 1), conflict-free for the
// 16-row ds_read_b128 fragment reads and for the 4-row x 2-chunk transposing reads.
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
template <int D>
__device__ __forceinline__ int toff(int r, int c) {
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

// Two floats to packed bf16, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t cvt2(float a, float b) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const bf16x2 v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}

// Score registers e0..e0+7 as a bf16 k-operand.
__device__ __forceinline__ bf16x8 pack8(const float* v) {
  u32x4 u;
#pragma unroll
  for (int w = 0; w < 4; ++w) u[w] = cvt2(v[2 * w], v[2 * w + 1]);
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
  const int j = threadIdx.x & 15;
  const int cpr = D / 8;  // 16-byte chunks per head row (8 or 16)
  float acc = 0.f;
  if (r < rows && j < cpr) {
    const int64_t t = r / Hl, head = r % Hl;
    const int64_t off = t * (int64_t)Hl * D + head * D + j * 8;
    const u32x4 a = *reinterpret_cast<const u32x4*>(dO + off);
    const u32x4 b = *reinterpret_cast<const u32x4*>(O + off);
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      acc += bf16_bits_to_f32(a[w] & 0xffffu) * bf16_bits_to_f32(b[w] & 0xffffu);
      acc += bf16_bits_to_f32(a[w] >> 16) * bf16_bits_to_f32(b[w] >> 16);
    }
  }
#pragma unroll
  for (int o = 8; o > 0; o >>= 1) acc += __shfl_xor(acc, o, 16);
  if (r < rows && j == 0) {
    const int64_t t = r / Hl, head = r % Hl, bi = t / s, q = t % s;
    Dout[(bi * Hl + head) * s + q] = acc;
  }
}

// ------------------------------------------------------------------ dK, dV
template <int D, bool CAUSAL, int NW>
__global__ __launch_bounds__(NW * 64) void dkdv_kernel(const uint16_t* __restrict__ qkv,
                                                       const uint16_t* __restrict__ dO,
                                                       const float* __restrict__ lse,
                                                       const float* __restrict__ Dv, uint16_t* __restrict__ dqkv,
                                                       int s, int Hl, int nkb, float scale_log2, float scale) {
  constexpr int NTH = NW * 64, KB = 32 * NW, KS = D / 16, DT = D / 32;
  constexpr int QP = 32 * D / 8 / NTH;  // 16-byte chunks per thread per 32-row tile
  __shared__ __attribute__((aligned(16))) uint16_t sK[KB * D];
  __shared__ __attribute__((aligned(16))) uint16_t sV[KB * D];
  __shared__ __attribute__((aligned(16))) uint16_t sQ[2][32 * D];
  __shared__ __attribute__((aligned(16))) uint16_t sdO[2][32 * D];
  __shared__ __attribute__((aligned(16))) float sL[2][32];
  __shared__ __attribute__((aligned(16))) float sDv[2][32];

  const int item = blockIdx.x;
  const int bh = item / nkb, kb = item % nkb;  // key block 0 (the heaviest) first
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
  const int qstart = CAUSAL ? k0 : 0;  // query blocks of 32 from the diagonal
  const int nq = (s - qstart + 31) / 32;
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
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const float4 L = *reinterpret_cast<const float4*>(&sL[buf][8 * g + 4 * hh]);
        const float4 Dd = *reinterpret_cast<const float4*>(&sDv[buf][8 * g + 4 * hh]);
        const float Lv[4] = {L.x, L.y, L.z, L.w}, Dq[4] = {Dd.x, Dd.y, Dd.z, Dd.w};
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const int e = 4 * g + c, q = q0 + 8 * g + 4 * hh + c;
          float pv = __builtin_amdgcn_exp2f(__builtin_fmaf(S[e], scale_log2, -Lv[c]));
          if ((CAUSAL && key > q) || key >= s) pv = 0.f;
          p[e] = pv;
          ds[e] = pv * (dP[e] - Dq[c]);
        }
      }
      const bf16x8 pa[2] = {pack8(p), pack8(p + 8)};
      const bf16x8 sa[2] = {pack8(ds), pack8(ds + 8)};
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int i = 0; i < DT; ++i) {
          dv[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pa[t], frag_tr<D>(td, 16 * t, 32 * i, lane), dv[i], 0, 0, 0);
          dk[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(sa[t], frag_tr<D>(tq, 16 * t, 32 * i, lane), dk[i], 0, 0, 0);
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
__global__ __launch_bounds__(NW * 64) void dq_kernel(const uint16_t* __restrict__ qkv, const uint16_t* __restrict__ dO,
                                                     const float* __restrict__ lse, const float* __restrict__ Dv,
                                                     uint16_t* __restrict__ dqkv, int s, int Hl, int nqb,
                                                     float scale_log2, float scale) {
  constexpr int NTH = NW * 64, QB = 32 * NW, KS = D / 16, DT = D / 32;
  constexpr int KP = 32 * D / 8 / NTH;
  __shared__ __attribute__((aligned(16))) uint16_t sK[2][32 * D];
  __shared__ __attribute__((aligned(16))) uint16_t sV[2][32 * D];

  const int item = blockIdx.x;
  const int bh = item / nqb, qb = nqb - 1 - item % nqb;  // the heaviest (last) query block first
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

  const int kend = CAUSAL ? min(s, q0 + QB) : s;
  const int nk = (kend + 31) / 32;
  u32x4 rk0[KP], rv0[KP], rk1[KP], rv1[KP];
  if (nk > 0) {
    load_rows<D, 32, NTH>(rk0, Kg, ld, 0, s, tid);
    load_rows<D, 32, NTH>(rv0, Vg, ld, 0, s, tid);
  }
  if (nk > 1) {
    load_rows<D, 32, NTH>(rk1, Kg, ld, 32, s, tid);
    load_rows<D, 32, NTH>(rv1, Vg, ld, 32, s, tid);
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
    const int k0 = 32 * j, buf = j & 1;
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
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int key = k0 + 8 * (e >> 2) + 4 * hh + (e & 3);
        float pv = __builtin_amdgcn_exp2f(__builtin_fmaf(S[e], scale_log2, -Lq));
        if ((CAUSAL && key > qrow) || key >= s) pv = 0.f;
        ds[e] = pv * (dP[e] - Dq);
      }
      const bf16x8 sa[2] = {pack8(ds), pack8(ds + 8)};
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int i = 0; i < DT; ++i)
          dq[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(frag_tr<D>(tk, 16 * t, 32 * i, lane), sa[t], dq[i], 0, 0, 0);
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
  if (qrow < s) {
    uint16_t* dQg = dqkv + ((int64_t)bi * s + qrow) * ld + (int64_t)head * D;
#pragma unroll
    for (int i = 0; i < DT; ++i)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        uint2 u;
        u.x = cvt2(dq[i][4 * g] * scale, dq[i][4 * g + 1] * scale);
        u.y = cvt2(dq[i][4 * g + 2] * scale, dq[i][4 * g + 3] * scale);
        *reinterpret_cast<uint2*>(dQg + 32 * i + 8 * g + 4 * hh) = u;
      }
  }
}

template <int D, bool C>
hipError_t launch_bwd(const uint16_t* qkv, const uint16_t* O, const uint16_t* dO, const float* lse, uint16_t* dqkv,
                      float* Dws, int b, int s, int Hl, hipStream_t st) {
  constexpr int NWK = 4, NWQ = 4;
  const int64_t rows = (int64_t)b * s * Hl;
  if (rows == 0) return hipSuccess;
  const float scale = 1.f / sqrtf((float)D), scale_log2 = kLog2e * scale;
  hipLaunchKernelGGL(rowdot_kernel, dim3((unsigned)((rows + 15) / 16)), dim3(256), 0, st, dO, O, Dws, s, Hl, D, rows);
  const int nkb = (s + 32 * NWK - 1) / (32 * NWK), nqb = (s + 32 * NWQ - 1) / (32 * NWQ);
  hipLaunchKernelGGL((dkdv_kernel<D, C, NWK>), dim3((unsigned)((int64_t)b * Hl * nkb)), dim3(NWK * 64), 0, st, qkv,
                     dO, lse, Dws, dqkv, s, Hl, nkb, scale_log2, scale);
  hipLaunchKernelGGL((dq_kernel<D, C, NWQ>), dim3((unsigned)((int64_t)b * Hl * nqb)), dim3(NWQ * 64), 0, st, qkv, dO,
                     lse, Dws, dqkv, s, Hl, nqb, scale_log2, scale);
  return hipGetLastError();
}

}  // namespace

hipError_t attn_bwd(const uint16_t* qkv, const uint16_t* O, const uint16_t* dO, const float* lse, uint16_t* dqkv,
                    float* Dws, int b, int s, int Hl, int d, bool causal, hipStream_t st) {
  if (d == 128)
    return causal ? launch_bwd<128, true>(qkv, O, dO, lse, dqkv, Dws, b, s, Hl, st)
                  : launch_bwd<128, false>(qkv, O, dO, lse, dqkv, Dws, b, s, Hl, st);
  if (d == 64)
    return causal ? launch_bwd<64, true>(qkv, O, dO, lse, dqkv, Dws, b, s, Hl, st)
                  : launch_bwd<64, false>(qkv, O, dO, lse, dqkv, Dws, b, s, Hl, st);
  return hipErrorInvalidValue;
}

}  // namespace tps
