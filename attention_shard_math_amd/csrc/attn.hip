// Fused softmax attention over one rank's local heads (gfx950, bf16 MFMA).
//
// For each sequence and local head: O = softmax(Q K^T / sqrt(d)) V, causal or
// not, with the online (running max / running sum) softmax so the s x s score
// matrix never leaves registers.
//
// Work split: one 512-thread workgroup per (sequence, head, 128-query block).
// Waves 0-3 compute, 32 queries each, over every key of the block; waves 4-7
// only move data: they load the next 64-key stage from global memory into
// registers (buffer loads, which read as zero past the last key) and write it
// to LDS, K as [key][d] and V transposed to [d][key] through a register
// transpose, while the compute waves work on the current stages (four LDS
// slots, one barrier per stage). Each SIMD thus runs one compute wave, whose
// MFMAs and softmax arithmetic overlap with the other wave's loads and LDS
// writes.
//
// The compute wave is software-pipelined two stages deep: the P V product of
// stage i - 1 and the scores of stage i + 1 (whose K is already in LDS) are
// issued in the same basic block as the softmax of stage i, so the MFMA unit
// works on them while the VALU forms exp2 and the bf16 P of stage i. The
// order of every accumulation is unchanged, so the output is bit-identical to
// the unpipelined schedule.
//
// The compute wave forms the transposed scores S^T = K Q^T and the transposed
// output O^T = V^T P^T with v_mfma_f32_32x32x16_bf16, so that in both
// accumulators a lane owns one query column: the row max, row sum and the
// rescaling of O stay per lane (one exchange between the two 32-lane halves
// per stage), and P feeds the second product straight from registers. V^T rows
// keep each 16-key group in the order 0-3, 8-11, 4-7, 12-15 so that one 16-byte
// LDS read yields the 8 keys a P^T operand lane holds.
//
// The running maximum used as the exponent reference is only raised when a
// row's maximum exceeds it by more than kTau (log2 units); until then P is
// formed against the older reference (values up to 2^kTau) and O is not
// rescaled. Numerator and denominator share the reference, so the result is
// the same softmax up to rounding.
//
// The training variant (which also writes the log-sum-exp for the backward)
// feeds P to the P V product as two bf16 MFMA operands, P_hi = bf16(P) and
// P_lo = bf16(P - P_hi), so P enters the product with about 16 significant
// bits instead of 8: the stored O then rounds to the same bf16 value as the
// exact result in all but a small fraction of entries, which keeps the
// weight gradients formed from O (dWo = O^T dOut) within the bf16 bar.
//
// Causal stages wholly above a wave's queries are skipped. Workgroup i runs on
// XCD i % 8; each XCD takes a contiguous, head-major range of (head, query
// block) items, heaviest query block first, so the K and V of a head are read
// from one L2.
#include "attn.hpp"
#include "common.hpp"

namespace tps {
namespace {

constexpr int AQ = 128;   // queries per workgroup: 4 compute waves x 32
constexpr int KVB = 64;   // keys per LDS stage: 2 tiles of 32
constexpr int NT = 512;   // waves 0-3 compute, waves 4-7 load
constexpr int NP = 256;   // loader threads
constexpr float kNegInf = -__builtin_huge_valf();
constexpr float kTau = 8.0f;

// Exchange between lanes l and l ^ 32: max / sum of the two halves' values.
__device__ __forceinline__ float xhalf_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xhalf_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
// Returns x unchanged but hides its value from the optimizer, so address math
// built on it is redone where used instead of occupying registers throughout.
__device__ __forceinline__ int opaque(int x) {
  asm volatile("" : "+v"(x));
  return x;
}

// K stage rows [key][d]: 16-byte chunk c of row key sits at c ^ swz_k(key).
template <int D>
__device__ __forceinline__ int swz_k(int key) { return D == 128 ? (key & 15) : ((key >> 1) & 7); }
// V^T stage rows [d][key'] of 64 keys: 16-byte chunk c of row d sits at c ^ swz_v(d).
__device__ __forceinline__ int swz_v(int d) { return (d ^ (d >> 3)) & 7; }

template <int D, bool CAUSAL, bool SPLIT>
__global__ __launch_bounds__(NT) void attn_fwd_kernel(const uint16_t* __restrict__ qkv, uint16_t* __restrict__ O, int s,
                                                      int Hl, int nqb, int per_xcd, int n_items, float scale_log2,
                                                      float* __restrict__ lse) {
  constexpr int DCH = D / 8;                // 16-byte chunks per K row
  constexpr int KS = D / 16;                // k-steps of S^T over d
  constexpr int DT = D / 32;                // O^T tiles along d
  constexpr int KPER = KVB * DCH / NP;      // K chunks each loader thread stages
  constexpr int NVT = (KVB / 8) * (D / 4);  // V tasks of 8 keys x 4 d
  constexpr int SK = KVB * D;               // elements per K (and per V^T) stage
  static_assert(KPER >= 1 && NVT <= NP && NVT % 64 == 0, "stage shape");
  __shared__ __attribute__((aligned(16))) uint16_t smem[4 * 2 * SK];  // [slot][K | V^T], stage i in slot i % 4

  const int item = (int)(blockIdx.x & 7) * per_xcd + (int)(blockIdx.x >> 3);
  if (item >= n_items) return;
  const int bh = item / nqb, qb = nqb - 1 - item % nqb;
  const int tid = threadIdx.x, wave = tid >> 6;
  const int bi = bh / Hl, head = bh % Hl;
  const int64_t ld = 3LL * Hl * D;
  const uint16_t* Qg = qkv + (int64_t)bi * s * ld + (int64_t)head * D;
  const int q0 = qb * AQ;
  const int kv_end = CAUSAL ? min(s, q0 + AQ) : s;
  const int nkv = (kv_end + KVB - 1) / KVB;

  if (wave >= 4) {
    // ---------------- loader waves ----------------
    const int ptid = tid - (NT - NP);
    // Range of one sequence's K (or V) rows: a load past the last key returns zeros.
    // Each stage's descriptors start at its first key (the range shortened to
    // match), so the per-thread offsets below stay fixed for the whole walk and a
    // stage costs the loaders only scalar address arithmetic.
    const int seq_bytes = (s - 1) * (int)ld * 2 + D * 2;
    const int row_b = (int)ld * 2;
    const char* kbase = reinterpret_cast<const char*>(Qg + (int64_t)Hl * D);
    const char* vbase = reinterpret_cast<const char*>(Qg + 2LL * Hl * D);
    auto rsrc_at = [&](const char* base, int kv0) __attribute__((always_inline)) {
      return __builtin_amdgcn_make_buffer_rsrc((void*)(base + (int64_t)kv0 * row_b), (short)0,
                                               seq_bytes - kv0 * row_b, 0x00020000);
    };
    // K: chunk c = ptid + p * NP is 16 bytes of key c / DCH, stored at [key][d] with
    // the chunk swizzle. V: task (vd4, vg8) takes d = 4*vd4 .. 4*vd4+3 of the 8 keys
    // that V^T chunk vg8 holds, keys 16*(vg8/2) + 4*(vg8%2) + {0..3, 8..11}.
    const bool vtask = NVT == NP || ptid < NVT;
    const int vd4 = ptid % (D / 4), vg8 = ptid / (D / 4);
    int kg[KPER], kl[KPER], vg[8], vl[4];
#pragma unroll
    for (int p = 0; p < KPER; ++p) {
      const int c = ptid + p * NP, key = c / DCH, ch = c % DCH;
      kg[p] = key * row_b + ch * 16;
      kl[p] = key * D + ((ch ^ swz_k<D>(key)) << 3);
    }
#pragma unroll
    for (int kk = 0; kk < 8; ++kk)
      vg[kk] = (16 * (vg8 >> 1) + 4 * (vg8 & 1) + (kk & 3) + 8 * (kk >> 2)) * row_b + vd4 * 8;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int d = vd4 * 4 + r;
      vl[r] = d * KVB + ((vg8 ^ swz_v(d)) << 3);
    }
    u32x4 kreg[KPER];
    uint2 vreg[8];
    auto load_kv = [&](int kv0) __attribute__((always_inline)) {
      const __amdgpu_buffer_rsrc_t rk = rsrc_at(kbase, kv0);
#pragma unroll
      for (int p = 0; p < KPER; ++p)
        kreg[p] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rk, kg[p], 0, 0));
      if (vtask) {
        const __amdgpu_buffer_rsrc_t rv = rsrc_at(vbase, kv0);
#pragma unroll
        for (int kk = 0; kk < 8; ++kk)
          vreg[kk] = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(rv, vg[kk], 0, 0));
      }
    };
    auto store_kv = [&](int buf) __attribute__((always_inline)) {
      uint16_t* sK = smem + buf * 2 * SK;
      uint16_t* sV = sK + SK;
#pragma unroll
      for (int p = 0; p < KPER; ++p) *reinterpret_cast<u32x4*>(sK + kl[p]) = kreg[p];
      if (vtask) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          u32x4 w;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const uint32_t a = (r < 2) ? vreg[2 * j].x : vreg[2 * j].y;
            const uint32_t b = (r < 2) ? vreg[2 * j + 1].x : vreg[2 * j + 1].y;
            w[j] = __builtin_amdgcn_perm(b, a, (r & 1) ? 0x07060302u : 0x05040100u);
          }
          *reinterpret_cast<u32x4*>(sV + vl[r]) = w;
        }
      }
    };
    // Stages 0 and 1 are in LDS before the compute waves start; during the
    // compute waves' stage i the loaders write stage i + 2 and fetch stage i + 3.
    load_kv(0);
    store_kv(0);
    if (nkv > 1) {
      load_kv(KVB);
      store_kv(1);
    }
    if (nkv > 2) load_kv(2 * KVB);
    __syncthreads();
    for (int it = 0; it < nkv; ++it) {
      if (it + 2 < nkv) store_kv((it + 2) % 4);
      if (it + 3 < nkv) load_kv((it + 3) * KVB);
      __syncthreads();
    }
    return;
  }

  // ---------------- compute waves ----------------
  const int lane = tid & 63, qg = wave;
  const int hh = lane >> 5, lr = lane & 31;
  const int qw = q0 + qg * 32, qrow = qw + lr;

  // Q^T fragments (B operand of S^T = K Q^T): query qrow, d chunk 2*ks + hh.
  bf16x8 qf[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    u32x4 v = {0u, 0u, 0u, 0u};
    if (qrow < s) v = *reinterpret_cast<const u32x4*>(Qg + (int64_t)qrow * ld + (2 * ks + hh) * 8);
    qf[ks] = __builtin_bit_cast(bf16x8, v);
  }
  f32x16 ot[DT];
#pragma unroll
  for (int i = 0; i < DT; ++i)
#pragma unroll
    for (int e = 0; e < 16; ++e) ot[i][e] = 0.f;
  float m_i = kNegInf;  // exponent reference of the row (scaled scores, log2 units)
  float l_i = 0.f;      // this lane-half's share of the row sum

  // S^T = K Q^T of one stage (two 32-key tiles), K fragments read as used.
  auto scores = [&](const uint16_t* sK, f32x16(&st)[2]) __attribute__((always_inline)) {
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int e = 0; e < 16; ++e) st[t][e] = 0.f;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const int kr = 32 * t + lr;
        const bf16x8 kf = *reinterpret_cast<const bf16x8*>(sK + kr * D + (((2 * ks + hh) ^ swz_k<D>(kr)) << 3));
        st[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[ks], st[t], 0, 0, 0);
      }
  };

  // O^T += V^T P^T of one stage over its 16-key groups 2t + s2; P^T lane (lr, hh)
  // holds keys {4hh + 0..3, 8 + 4hh + 0..3} of the group = V^T chunk 2(2t + s2) + hh.
  auto pv = [&](const uint16_t* sV, const bf16x8(&pb)[2][2], const bf16x8(&pl)[2][2]) __attribute__((always_inline)) {
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
        for (int i = 0; i < DT; ++i) {
          const int d = 32 * i + lr;
          const bf16x8 vf = *reinterpret_cast<const bf16x8*>(sV + d * KVB + (((4 * t + 2 * s2 + hh) ^ swz_v(d)) << 3));
          ot[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pb[t][s2], ot[i], 0, 0, 0);
          if constexpr (SPLIT) ot[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pl[t][s2], ot[i], 0, 0, 0);
        }
  };

  // Software pipeline, two stages deep: one basic block holds the softmax of stage
  // i (VALU), the P V product of stage i - 1 and the scores of stage i + 1 (MFMA),
  // so the MFMA unit works while the VALU forms the exponentials. The stage's K and
  // V sit in LDS slot i % 4: K(i + 1) and V(i - 1) are read while the loaders write
  // stage i + 2. When stage i raises the exponent reference, O (then summed through
  // stage i - 1) is rescaled at the top of the next step, before the P V product of
  // stage i: every accumulation keeps the order of the one-stage schedule.
  f32x16 sc[2];
  bf16x8 pp[2][2], ppl[2][2];  // P of the previous stage (hi, lo); zeros before stage 0
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) pp[t][s2] = ppl[t][s2] = bf16x8{};
  bool pending = false;     // wave-uniform: the previous stage's P V product is still to run
  bool rescale = false;     // wave-uniform: O is to be scaled by alpha_prev first
  float alpha_prev = 1.f;
  __syncthreads();
  scores(smem, sc);
  for (int it = 0; it < nkv; ++it) {
    const int kv0 = it * KVB;
    if (rescale) {
#pragma unroll
      for (int i = 0; i < DT; ++i)
#pragma unroll
        for (int e = 0; e < 16; ++e) ot[i][e] *= alpha_prev;
      rescale = false;
    }
    // V of the previous stage (before stage 0: stage 0's V, multiplied by zero P)
    const uint16_t* sVp = smem + (it == 0 ? 0 : (it + 3) % 4) * 2 * SK + SK;
    const uint16_t* sKn = smem + ((it + 1) % 4) * 2 * SK;  // K of the next stage
    // Wave-uniform: skip the stage if its first key is above the diagonal. Such stages
    // only follow the wave's last live one. (Every stage of the walk starts below s.)
    if (!(CAUSAL && kv0 > qw)) {
      // S^T accumulator lane (lr, hh), reg e of tile t: key kv0 + 32t + 8(e/4) + 4hh + e%4, query qrow.
      if ((CAUSAL && kv0 + KVB - 1 > qw) || kv0 + KVB > s) {
        // key - (kv0 + 4hh) = 32t + 8(e/4) + e%4 may not exceed lim.
        const int lim = (CAUSAL ? min(qrow, s - 1) : s - 1) - kv0 - 4 * hh;
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int e = 0; e < 16; ++e)
            if (32 * t + 8 * (e >> 2) + (e & 3) > lim) sc[t][e] = kNegInf;
      }
      float mx = fmaxf(sc[0][0], sc[1][0]);
#pragma unroll
      for (int e = 1; e < 16; ++e) mx = fmaxf(mx, fmaxf(sc[0][e], sc[1][e]));
      const float mt = xhalf_max(mx) * scale_log2;
      // Raise the reference only when some row's maximum has passed it by more
      // than kTau; rows that have not keep their reference (factor 1).
      const bool raise = __builtin_amdgcn_ballot_w64(mt > m_i + kTau) != 0;
      const float mn = raise ? fmaxf(m_i, mt) : m_i;
      const float alpha = (mn == kNegInf) ? 1.f : __builtin_amdgcn_exp2f(m_i - mn);
      l_i = raise ? l_i * alpha : l_i;
      m_i = mn;
      const float mref = m_i == kNegInf ? 0.f : m_i;
      float rs = 0.f;
      bf16x8 pb[2][2], pl[2][2];
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
          u32x4 u, ul;
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[t][8 * s2 + 2 * w], scale_log2, -mref));
            const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[t][8 * s2 + 2 * w + 1], scale_log2, -mref));
            rs += p0 + p1;
            u[w] = pack_bf16x2(p0, p1);
            if constexpr (SPLIT)
              ul[w] = pack_bf16x2(p0 - bf16_bits_to_f32(u[w] & 0xffffu), p1 - bf16_bits_to_f32(u[w] >> 16));
          }
          pb[t][s2] = __builtin_bit_cast(bf16x8, u);
          if constexpr (SPLIT) pl[t][s2] = __builtin_bit_cast(bf16x8, ul);
        }
      pv(sVp, pp, ppl);
      f32x16 sn[2];
      scores(sKn, sn);
      sc[0] = sn[0];
      sc[1] = sn[1];
      l_i += rs;
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
          pp[t][s2] = pb[t][s2];
          if constexpr (SPLIT) ppl[t][s2] = pl[t][s2];
        }
      pending = true;
      rescale = raise;
      alpha_prev = alpha;
    } else if (pending) {
      pv(sVp, pp, ppl);
      pending = false;
    }
    __syncthreads();
  }
  // the last live stage's P V product (its V is still in its slot: the loaders are done)
  if (rescale) {
#pragma unroll
    for (int i = 0; i < DT; ++i)
#pragma unroll
      for (int e = 0; e < 16; ++e) ot[i][e] *= alpha_prev;
  }
  if (pending) pv(smem + ((nkv - 1) % 4) * 2 * SK + SK, pp, ppl);

  if (qrow < s) {
    const int ln = opaque(lane), lr2 = ln & 31, hh2 = ln >> 5;
    const float lsum = xhalf_sum(l_i);
    const float inv = 1.f / lsum;
    if (lse && hh2 == 0) {
      // natural-log log-sum-exp of the row's scaled scores: (m + log2 l) * ln 2
      const float mref = m_i == kNegInf ? 0.f : m_i;
      lse[((int64_t)bi * Hl + head) * s + qw + lr2] = (mref + __log2f(lsum)) * 0.69314718055994531f;
    }
    uint16_t* orow = O + ((int64_t)bi * s + qw + lr2) * ((int64_t)Hl * D) + (int64_t)head * D;
    // O^T accumulator lane (lr, hh), reg e of tile i: d = 32i + 8(e/4) + 4hh + e%4.
#pragma unroll
    for (int i = 0; i < DT; ++i)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        uint2 u;
        u.x = pack_bf16x2(ot[i][4 * g] * inv, ot[i][4 * g + 1] * inv);
        u.y = pack_bf16x2(ot[i][4 * g + 2] * inv, ot[i][4 * g + 3] * inv);
        *reinterpret_cast<uint2*>(orow + 32 * i + 8 * g + 4 * hh2) = u;
      }
  }
}

// ---------------------------------------------------------------- wide heads
// Heads of d = 384 (h = 18432 over 48 heads): three LDS slots of a 64-key stage
// would take 288 KB, and a compute wave cannot hold a 384-wide O^T next to its
// Q^T fragments. So the output is split into chunks of WDC = 128 columns: one
// workgroup per (sequence, head, 128-query block, d-chunk). Each forms the full
// scores S^T = K Q^T over all 384 d (the K stage is [64 keys][384]) and only
// its chunk's O^T = V_c^T P^T, so S is formed once per chunk (three times per
// query block). Two LDS slots of 64 KB (K stage + the chunk's V^T stage), one
// barrier per stage; during stage i the loaders write stage i + 1 and fetch
// stage i + 2. The three chunks of one query block are adjacent items on one XCD,
// so their K and V stages are read from one L2. Softmax, masking, the exponent
// reference and the hi/lo split of P are as in attn_fwd_kernel.
constexpr int WD = 384, WDC = 128, WNC = WD / WDC;

template <bool CAUSAL, bool SPLIT>
__global__ __launch_bounds__(NT) void attn_fwd_wide_kernel(const uint16_t* __restrict__ qkv, uint16_t* __restrict__ O,
                                                           int s, int Hl, int nqb, int per_xcd, int n_items,
                                                           float scale_log2, float* __restrict__ lse) {
  constexpr int D = WD, DC = WDC;
  constexpr int DCH = D / 8;                 // 16-byte chunks per K row (48)
  constexpr int KS = D / 16;                 // k-steps of S^T over d (24)
  constexpr int DT = DC / 32;                // O^T tiles of the chunk (4)
  constexpr int KPER = KVB * DCH / NP;       // K chunks each loader thread stages (12)
  constexpr int NVT = (KVB / 8) * (DC / 4);  // V tasks of 8 keys x 4 d (256)
  constexpr int SKK = KVB * D;               // elements of a K stage
  constexpr int SVV = KVB * DC;              // elements of a V^T chunk stage
  static_assert(KPER * NP == KVB * DCH && NVT == NP, "stage shape");
  __shared__ __attribute__((aligned(16))) uint16_t smem[2 * (SKK + SVV)];  // [slot][K | V^T], stage i in slot i % 2

  const int item = (int)(blockIdx.x & 7) * per_xcd + (int)(blockIdx.x >> 3);
  if (item >= n_items) return;
  const int per_bh = nqb * WNC;
  const int bh = item / per_bh, rem = item % per_bh;
  const int qb = nqb - 1 - rem / WNC, dc = rem % WNC;
  const int tid = threadIdx.x, wave = tid >> 6;
  const int bi = bh / Hl, head = bh % Hl;
  const int64_t ld = 3LL * Hl * D;
  const uint16_t* Qg = qkv + (int64_t)bi * s * ld + (int64_t)head * D;
  const int q0 = qb * AQ;
  const int kv_end = CAUSAL ? min(s, q0 + AQ) : s;
  const int nkv = (kv_end + KVB - 1) / KVB;

  if (wave >= 4) {
    // ---------------- loader waves ----------------
    const int ptid = tid - (NT - NP);
    // As in attn_fwd_kernel: each stage's descriptors start at its first key, the
    // per-thread offsets stay fixed. V is the chunk's 128 columns.
    const int seq_bytes = (s - 1) * (int)ld * 2 + D * 2;
    const int row_b = (int)ld * 2;
    const char* kbase = reinterpret_cast<const char*>(Qg + (int64_t)Hl * D);
    const char* vbase = reinterpret_cast<const char*>(Qg + 2LL * Hl * D + dc * DC);
    const int vbytes = seq_bytes - dc * DC * 2;
    const int vd4 = ptid % (DC / 4), vg8 = ptid / (DC / 4);
    int kg[KPER], kl[KPER], vg[8], vl[4];
#pragma unroll
    for (int p = 0; p < KPER; ++p) {
      const int c = ptid + p * NP, key = c / DCH, ch = c % DCH;
      kg[p] = key * row_b + ch * 16;
      kl[p] = key * D + ((ch ^ (key & 15)) << 3);
    }
#pragma unroll
    for (int kk = 0; kk < 8; ++kk)
      vg[kk] = (16 * (vg8 >> 1) + 4 * (vg8 & 1) + (kk & 3) + 8 * (kk >> 2)) * row_b + vd4 * 8;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int d = vd4 * 4 + r;
      vl[r] = d * KVB + ((vg8 ^ swz_v(d)) << 3);
    }
    u32x4 kreg[KPER];
    uint2 vreg[8];
    auto load_kv = [&](int kv0) __attribute__((always_inline)) {
      const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
          (void*)(kbase + (int64_t)kv0 * row_b), (short)0, seq_bytes - kv0 * row_b, 0x00020000);
      const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
          (void*)(vbase + (int64_t)kv0 * row_b), (short)0, vbytes - kv0 * row_b, 0x00020000);
#pragma unroll
      for (int p = 0; p < KPER; ++p)
        kreg[p] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rk, kg[p], 0, 0));
#pragma unroll
      for (int kk = 0; kk < 8; ++kk)
        vreg[kk] = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(rv, vg[kk], 0, 0));
    };
    auto store_kv = [&](int buf) __attribute__((always_inline)) {
      uint16_t* sK = smem + buf * (SKK + SVV);
      uint16_t* sV = sK + SKK;
#pragma unroll
      for (int p = 0; p < KPER; ++p) *reinterpret_cast<u32x4*>(sK + kl[p]) = kreg[p];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        u32x4 w;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const uint32_t a = (r < 2) ? vreg[2 * j].x : vreg[2 * j].y;
          const uint32_t b = (r < 2) ? vreg[2 * j + 1].x : vreg[2 * j + 1].y;
          w[j] = __builtin_amdgcn_perm(b, a, (r & 1) ? 0x07060302u : 0x05040100u);
        }
        *reinterpret_cast<u32x4*>(sV + vl[r]) = w;
      }
    };
    load_kv(0);
    store_kv(0);
    if (nkv > 1) load_kv(KVB);
    __syncthreads();
    for (int it = 0; it < nkv; ++it) {
      if (it + 1 < nkv) store_kv((it + 1) & 1);
      if (it + 2 < nkv) load_kv((it + 2) * KVB);
      __syncthreads();
    }
    return;
  }

  // ---------------- compute waves ----------------
  const int lane = tid & 63, qg = wave;
  const int hh = lane >> 5, lr = lane & 31;
  const int qw = q0 + qg * 32, qrow = qw + lr;
  bf16x8 qf[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    u32x4 v = {0u, 0u, 0u, 0u};
    if (qrow < s) v = *reinterpret_cast<const u32x4*>(Qg + (int64_t)qrow * ld + (2 * ks + hh) * 8);
    qf[ks] = __builtin_bit_cast(bf16x8, v);
  }
  f32x16 ot[DT];
#pragma unroll
  for (int i = 0; i < DT; ++i)
#pragma unroll
    for (int e = 0; e < 16; ++e) ot[i][e] = 0.f;
  float m_i = kNegInf, l_i = 0.f;

  __syncthreads();
  for (int it = 0; it < nkv; ++it) {
    const int kv0 = it * KVB;
    const uint16_t* sK = smem + (it & 1) * (SKK + SVV);
    const uint16_t* sV = sK + SKK;
    if (!((CAUSAL && kv0 > qw) || kv0 >= s)) {
      f32x16 sc[2];
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int e = 0; e < 16; ++e) sc[t][e] = 0.f;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const int kr = 32 * t + lr;
          const bf16x8 kf = *reinterpret_cast<const bf16x8*>(sK + kr * D + (((2 * ks + hh) ^ (kr & 15)) << 3));
          sc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[ks], sc[t], 0, 0, 0);
        }
      if ((CAUSAL && kv0 + KVB - 1 > qw) || kv0 + KVB > s) {
        const int lim = (CAUSAL ? min(qrow, s - 1) : s - 1) - kv0 - 4 * hh;
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int e = 0; e < 16; ++e)
            if (32 * t + 8 * (e >> 2) + (e & 3) > lim) sc[t][e] = kNegInf;
      }
      float mx = fmaxf(sc[0][0], sc[1][0]);
#pragma unroll
      for (int e = 1; e < 16; ++e) mx = fmaxf(mx, fmaxf(sc[0][e], sc[1][e]));
      const float mt = xhalf_max(mx) * scale_log2;
      if (__builtin_amdgcn_ballot_w64(mt > m_i + kTau) != 0) {
        const float mn = fmaxf(m_i, mt);
        const float alpha = (mn == kNegInf) ? 1.f : __builtin_amdgcn_exp2f(m_i - mn);
        l_i *= alpha;
#pragma unroll
        for (int i = 0; i < DT; ++i)
#pragma unroll
          for (int e = 0; e < 16; ++e) ot[i][e] *= alpha;
        m_i = mn;
      }
      const float mref = m_i == kNegInf ? 0.f : m_i;
      float rs = 0.f;
      bf16x8 pb[2][2], pl[2][2];
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
          u32x4 u, ul;
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[t][8 * s2 + 2 * w], scale_log2, -mref));
            const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[t][8 * s2 + 2 * w + 1], scale_log2, -mref));
            rs += p0 + p1;
            u[w] = pack_bf16x2(p0, p1);
            if constexpr (SPLIT)
              ul[w] = pack_bf16x2(p0 - bf16_bits_to_f32(u[w] & 0xffffu), p1 - bf16_bits_to_f32(u[w] >> 16));
          }
          pb[t][s2] = __builtin_bit_cast(bf16x8, u);
          if constexpr (SPLIT) pl[t][s2] = __builtin_bit_cast(bf16x8, ul);
        }
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
          for (int i = 0; i < DT; ++i) {
            const int d = 32 * i + lr;
            const bf16x8 vf = *reinterpret_cast<const bf16x8*>(sV + d * KVB + (((4 * t + 2 * s2 + hh) ^ swz_v(d)) << 3));
            ot[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pb[t][s2], ot[i], 0, 0, 0);
            if constexpr (SPLIT) ot[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pl[t][s2], ot[i], 0, 0, 0);
          }
      l_i += rs;
    }
    __syncthreads();
  }

  if (qrow < s) {
    const int ln = opaque(lane), lr2 = ln & 31, hh2 = ln >> 5;
    const float lsum = xhalf_sum(l_i);
    const float inv = 1.f / lsum;
    if (lse && dc == 0 && hh2 == 0) {
      const float mref = m_i == kNegInf ? 0.f : m_i;
      lse[((int64_t)bi * Hl + head) * s + qw + lr2] = (mref + __log2f(lsum)) * 0.69314718055994531f;
    }
    uint16_t* orow = O + ((int64_t)bi * s + qw + lr2) * ((int64_t)Hl * D) + (int64_t)head * D + dc * DC;
#pragma unroll
    for (int i = 0; i < DT; ++i)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        uint2 u;
        u.x = pack_bf16x2(ot[i][4 * g] * inv, ot[i][4 * g + 1] * inv);
        u.y = pack_bf16x2(ot[i][4 * g + 2] * inv, ot[i][4 * g + 3] * inv);
        *reinterpret_cast<uint2*>(orow + 32 * i + 8 * g + 4 * hh2) = u;
      }
  }
}

template <bool C, bool SPLIT>
hipError_t launch_attn_wide(const uint16_t* qkv, uint16_t* O, float* lse, int b, int s, int Hl, hipStream_t st) {
  const int nqb = (s + AQ - 1) / AQ;
  const int64_t items = (int64_t)b * Hl * nqb * WNC;
  if (items == 0) return hipSuccess;
  // Buffer offsets are 32-bit: the furthest key row read is s - 1 + 1 stage.
  if (items > (1LL << 28) || (int64_t)(s + 2 * KVB) * 3 * Hl * WD * 2 >= (1LL << 31)) return hipErrorInvalidValue;
  const int per_xcd = (int)((items + 7) / 8);
  const float scale_log2 = 1.4426950408889634f / sqrtf((float)WD);
  hipLaunchKernelGGL((attn_fwd_wide_kernel<C, SPLIT>), dim3(8u * per_xcd), dim3(NT), 0, st, qkv, O, s, Hl, nqb,
                     per_xcd, (int)items, scale_log2, lse);
  return hipGetLastError();
}

template <int D, bool C, bool SPLIT>
hipError_t launch_attn(const uint16_t* qkv, uint16_t* O, float* lse, int b, int s, int Hl, hipStream_t st) {
  const int nqb = (s + AQ - 1) / AQ;
  const int64_t items = (int64_t)b * Hl * nqb;
  if (items == 0) return hipSuccess;
  // Buffer offsets are 32-bit: the furthest key row read is s - 1 + 2 stages.
  if (items > (1LL << 28) || (int64_t)(s + 2 * KVB) * 3 * Hl * D * 2 >= (1LL << 31)) return hipErrorInvalidValue;
  const int per_xcd = (int)((items + 7) / 8);
  const float scale_log2 = 1.4426950408889634f / sqrtf((float)D);
  hipLaunchKernelGGL((attn_fwd_kernel<D, C, SPLIT>), dim3(8u * per_xcd), dim3(NT), 0, st, qkv, O, s, Hl, nqb, per_xcd,
                     (int)items, scale_log2, lse);
  return hipGetLastError();
}

template <int D>
hipError_t attn_fwd_d(const uint16_t* qkv, uint16_t* O, int b, int s, int Hl, bool causal, hipStream_t st,
                      float* lse) {
  // with lse (training) P enters the P V product as a hi/lo bf16 pair
  if (lse)
    return causal ? launch_attn<D, true, true>(qkv, O, lse, b, s, Hl, st)
                  : launch_attn<D, false, true>(qkv, O, lse, b, s, Hl, st);
  return causal ? launch_attn<D, true, false>(qkv, O, lse, b, s, Hl, st)
                : launch_attn<D, false, false>(qkv, O, lse, b, s, Hl, st);
}

}  // namespace

hipError_t attn_fwd(const uint16_t* qkv, uint16_t* O, int b, int s, int Hl, int d, bool causal, hipStream_t st,
                    float* lse) {
  if (d == 128) return attn_fwd_d<128>(qkv, O, b, s, Hl, causal, st, lse);
  if (d == 64) return attn_fwd_d<64>(qkv, O, b, s, Hl, causal, st, lse);
  if (d == WD) {
    if (lse)
      return causal ? launch_attn_wide<true, true>(qkv, O, lse, b, s, Hl, st)
                    : launch_attn_wide<false, true>(qkv, O, lse, b, s, Hl, st);
    return causal ? launch_attn_wide<true, false>(qkv, O, lse, b, s, Hl, st)
                  : launch_attn_wide<false, false>(qkv, O, lse, b, s, Hl, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace tps
