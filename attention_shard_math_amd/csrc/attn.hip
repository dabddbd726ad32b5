// Fused softmax attention over one rank's local heads (gfx950, bf16 MFMA).
//
// For each sequence and local head: O = softmax(Q K^T / sqrt(d)) V, causal or
// not, with the online (running max / running sum) softmax so the s x s score
// matrix never leaves registers.
//
// Work split: one 256-thread workgroup per (sequence, head, 128-query block);
// each of its 4 waves owns 32 queries. Key/value blocks of 64 keys are staged in
// LDS (double-buffered, the next block's global loads in flight during the
// current block's MFMAs): K as [key][d] and V transposed to [d][key] through an
// 8x8 register transpose. The kernel computes the transposed scores
// S^T = K Q^T and the transposed output O^T = V^T P^T with
// v_mfma_f32_32x32x16_bf16, so that in both accumulators a lane owns one query
// column: the row max, row sum and the rescaling of O stay per lane (one
// cross-half exchange per block), and P feeds the second product straight from
// registers. Causal blocks wholly above a wave's queries are skipped; the
// heaviest query blocks are scheduled first.
#include "attn.hpp"
#include "common.hpp"

namespace tps {
namespace {

constexpr int AQ = 128;  // queries per workgroup
constexpr int AKV = 64;  // keys per LDS block
constexpr float kNegInf = -__builtin_huge_valf();

__device__ __forceinline__ int swz8(int row) { return (row ^ (row >> 3)) & 7; }

template <int D, bool CAUSAL>
__global__ __launch_bounds__(256) void attn_fwd_kernel(const uint16_t* __restrict__ qkv, uint16_t* __restrict__ O,
                                                       int b, int s, int Hl, float scale_log2) {
  constexpr int DCH = D / 8;           // 16-byte chunks per K row
  constexpr int KS = D / 16;           // MFMA k-steps over d
  constexpr int DT = D / 32;           // O^T tiles along d
  constexpr int KPER = AKV * DCH / 256;
  constexpr int VBLK = (AKV / 8) * (D / 8);
  static_assert(AKV * DCH % 256 == 0 && VBLK <= 256, "tile shape");

  __shared__ __attribute__((aligned(16))) uint16_t sK[2][AKV * D];  // [key][d]
  __shared__ __attribute__((aligned(16))) uint16_t sV[2][D * AKV];  // [d][key]

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int hh = lane >> 5, lr = lane & 31;
  const int nqb = (s + AQ - 1) / AQ;
  const int bh = blockIdx.x % (b * Hl);
  const int qb = nqb - 1 - (int)(blockIdx.x / (b * Hl));
  const int bi = bh / Hl, head = bh % Hl;
  const int64_t ld = 3LL * Hl * D;
  const uint16_t* Qg = qkv + (int64_t)bi * s * ld + (int64_t)head * D;
  const uint16_t* Kg = Qg + (int64_t)Hl * D;
  const uint16_t* Vg = Qg + 2LL * Hl * D;
  const int q0 = qb * AQ;
  const int qw = q0 + wave * 32;
  const int qrow = qw + lr;

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
  float m_i = kNegInf, l_i = 0.f;

  const int kv_end = CAUSAL ? min(s, q0 + AQ) : s;
  const int nkv = (kv_end + AKV - 1) / AKV;

  u32x4 kreg[KPER];
  u32x4 vreg[8];
  auto load_kv = [&](int kv0) {
#pragma unroll
    for (int p = 0; p < KPER; ++p) {
      const int c = tid + p * 256, r = c / DCH, ch = c % DCH, key = kv0 + r;
      kreg[p] = key < s ? *reinterpret_cast<const u32x4*>(Kg + (int64_t)key * ld + ch * 8) : u32x4{0u, 0u, 0u, 0u};
    }
    if (tid < VBLK) {
      const int kb = tid / (D / 8), db = tid % (D / 8);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int key = kv0 + kb * 8 + j;
        vreg[j] = key < s ? *reinterpret_cast<const u32x4*>(Vg + (int64_t)key * ld + db * 8) : u32x4{0u, 0u, 0u, 0u};
      }
    }
  };
  auto store_kv = [&](int buf) {
#pragma unroll
    for (int p = 0; p < KPER; ++p) {
      const int c = tid + p * 256, r = c / DCH, ch = c % DCH;
      *reinterpret_cast<u32x4*>(sK[buf] + r * D + ((ch ^ (r & (DCH - 1))) << 3)) = kreg[p];
    }
    if (tid < VBLK) {
      const int kb = tid / (D / 8), db = tid % (D / 8);
      // vreg[j] holds d = db*8 + 0..7 of key kb*8 + j; row d of V^T gathers
      // element d of each of the 8 keys.
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        u32x4 lo, hi;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const uint32_t a = vreg[2 * w][q], c = vreg[2 * w + 1][q];
          lo[w] = (a & 0xffffu) | (c << 16);
          hi[w] = (a >> 16) | (c & 0xffff0000u);
        }
        const int d0 = db * 8 + 2 * q;
        *reinterpret_cast<u32x4*>(sV[buf] + d0 * AKV + ((kb ^ swz8(d0)) << 3)) = lo;
        *reinterpret_cast<u32x4*>(sV[buf] + (d0 + 1) * AKV + ((kb ^ swz8(d0 + 1)) << 3)) = hi;
      }
    }
  };

  load_kv(0);
  store_kv(0);
  __syncthreads();

  for (int it = 0; it < nkv; ++it) {
    const int cur = it & 1, kv0 = it * AKV;
    if (it + 1 < nkv) load_kv(kv0 + AKV);
    const bool active = !CAUSAL || kv0 <= qw + 31;
    if (active) {
      const uint16_t* kS = sK[cur];
      const uint16_t* vS = sV[cur];
      // S^T block: 2 tiles of 32 keys x 32 queries. Accumulator lane l, reg e:
      // key 32t + 8*(e/4) + 4*hh + e%4, query lr.
      f32x16 st[2];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
#pragma unroll
        for (int e = 0; e < 16; ++e) st[t][e] = 0.f;
        const int kr = 32 * t + lr;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const bf16x8 kf = *reinterpret_cast<const bf16x8*>(kS + kr * D + (((2 * ks + hh) ^ (kr & (DCH - 1))) << 3));
          st[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[ks], st[t], 0, 0, 0);
        }
      }
      float mx = kNegInf;
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int key = kv0 + 32 * t + 8 * (e >> 2) + 4 * hh + (e & 3);
          float v = st[t][e] * scale_log2;
          if ((CAUSAL && key > qrow) || key >= s) v = kNegInf;
          st[t][e] = v;
          mx = fmaxf(mx, v);
        }
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float m_new = fmaxf(m_i, mx);
      const float m_use = (m_new == kNegInf) ? 0.f : m_new;
      const float alpha = exp2f(m_i - m_use);
      float rs = 0.f;
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const float p = exp2f(st[t][e] - m_use);
          st[t][e] = p;
          rs += p;
        }
      rs += __shfl_xor(rs, 32);
      l_i = l_i * alpha + rs;
      m_i = m_new;
#pragma unroll
      for (int i = 0; i < DT; ++i)
#pragma unroll
        for (int e = 0; e < 16; ++e) ot[i][e] *= alpha;
      // P^T as B operands: tile t, step s2 takes registers 8*s2 .. 8*s2+7, i.e.
      // keys 32t + 16*s2 + {4hh + 0..3, 8 + 4hh + 0..3}.
      bf16x8 pb[2][2];
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
          u32x4 u;
#pragma unroll
          for (int w = 0; w < 4; ++w) u[w] = pack_bf16x2(st[t][8 * s2 + 2 * w], st[t][8 * s2 + 2 * w + 1]);
          pb[t][s2] = __builtin_bit_cast(bf16x8, u);
        }
      // O^T += V^T P^T. A operand: d row 32i + lr, the same 8 keys as pb.
#pragma unroll
      for (int i = 0; i < DT; ++i) {
        const int d = 32 * i + lr;
        const uint16_t* vrow = vS + d * AKV;
        const int sw = swz8(d);
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int s2 = 0; s2 < 2; ++s2) {
            const int c0 = 4 * t + 2 * s2;
            const uint2 x0 = *reinterpret_cast<const uint2*>(vrow + ((c0 ^ sw) << 3) + 4 * hh);
            const uint2 x1 = *reinterpret_cast<const uint2*>(vrow + (((c0 + 1) ^ sw) << 3) + 4 * hh);
            const u32x4 u = {x0.x, x0.y, x1.x, x1.y};
            ot[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, u), pb[t][s2], ot[i], 0, 0, 0);
          }
      }
    }
    if (it + 1 < nkv) store_kv(cur ^ 1);
    __syncthreads();
  }

  // O^T accumulator: lane l, reg e holds d = 32i + 8*(e/4) + 4*hh + e%4 of query lr:
  // four consecutive d per register group -> one 8-byte store each.
  if (qrow < s) {
    const float inv = 1.f / l_i;
    uint16_t* orow = O + ((int64_t)bi * s + qrow) * ((int64_t)Hl * D) + (int64_t)head * D;
#pragma unroll
    for (int i = 0; i < DT; ++i)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        uint2 u;
        u.x = pack_bf16x2(ot[i][4 * g] * inv, ot[i][4 * g + 1] * inv);
        u.y = pack_bf16x2(ot[i][4 * g + 2] * inv, ot[i][4 * g + 3] * inv);
        *reinterpret_cast<uint2*>(orow + 32 * i + 8 * g + 4 * hh) = u;
      }
  }
}

template <int D, bool C>
hipError_t launch_attn(const uint16_t* qkv, uint16_t* O, int b, int s, int Hl, hipStream_t st) {
  const int nqb = (s + AQ - 1) / AQ;
  const int64_t blocks = (int64_t)b * Hl * nqb;
  if (blocks == 0) return hipSuccess;
  const float scale_log2 = 1.4426950408889634f / sqrtf((float)D);
  hipLaunchKernelGGL((attn_fwd_kernel<D, C>), dim3((unsigned)blocks), dim3(256), 0, st, qkv, O, b, s, Hl, scale_log2);
  return hipGetLastError();
}

}  // namespace

hipError_t attn_fwd(const uint16_t* qkv, uint16_t* O, int b, int s, int Hl, int d, bool causal, hipStream_t st) {
  if (d == 128) return causal ? launch_attn<128, true>(qkv, O, b, s, Hl, st) : launch_attn<128, false>(qkv, O, b, s, Hl, st);
  if (d == 64) return causal ? launch_attn<64, true>(qkv, O, b, s, Hl, st) : launch_attn<64, false>(qkv, O, b, s, Hl, st);
  return hipErrorInvalidValue;
}

}  // namespace tps
