// Device helpers shared by the gfx950 kernels of libtpshard: vector types,
// bfloat16 conversion, the erf-form GeLU and its derivative (with the device erff
// for float32 results, and from a published erfc fit for results rounded to bf16).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tps {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// float32 -> bfloat16 bits with gfx950's v_cvt_pk_bf16_f32: round to nearest, ties to
// even; a NaN stays a NaN.
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float x) {
  return __builtin_bit_cast(uint16_t, (__bf16)x);
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) {
  return __uint_as_float(b << 16);
}

// Two floats -> packed bf16 pair (lo in bits 0..15), one v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const bf16x2 v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

// GeLU(u) = u * Phi(u) = 0.5 u (1 + erf(u / sqrt 2)), with the device erff.
__device__ __forceinline__ float gelu_erf(float u) {
  return 0.5f * u * (1.0f + erff(u * 0.70710678118654752440f));
}

// GeLU'(u) = Phi(u) + u * phi(u).
__device__ __forceinline__ float gelu_erf_prime(float u) {
  const float cdf = 0.5f * (1.0f + erff(u * 0.70710678118654752440f));
  const float pdf = 0.39894228040143267794f * __expf(-0.5f * u * u);
  return cdf + u * pdf;
}

// Phi(u) and exp(-u^2/2) for epilogues whose results are rounded to bf16, from the
// rational-exponential fit of erfc in Abramowitz and Stegun, Handbook of Mathematical
// Functions, formula 7.1.26 (after Hastings): for x >= 0 and t = 1 / (1 + p x),
// erfc(x) = t (a1 + t (a2 + t (a3 + t (a4 + t a5)))) exp(-x^2) + e(x) with |e| <= 1.5e-7.
// With x = |u| / sqrt 2, exp(-x^2) = exp(-u^2/2); the coefficients below are the published
// a1..a5 halved, so the product is erfc(x) / 2 = Phi(-|u|). Phi(u) takes that value for
// u < 0 (the tail without cancellation) and 1 minus it otherwise. Evaluated in float32
// the error on Phi stays under 3e-7 (0.75e-7 from the fit, the rest from rounding in
// the alternating sum near u = 0), so GeLU and GeLU' are within 4e-7 max(1, |u|) of
// the exact erf form: below the bf16 rounding of the stored result wherever that is
// above ~1e-4 in magnitude. The bound is absolute: deep in the negative tail
// (u < -4, |GeLU(u)| < 1.3e-4) the relative error exceeds bf16 rounding.
struct PhiExp {
  float phi;  // Phi(u)
  float e;    // exp(-u^2 / 2)
};
__device__ __forceinline__ PhiExp phi_as7126(float u) {
  const float x = fabsf(u) * 0.70710678118654752440f;
  const float t = __builtin_amdgcn_rcpf(fmaf(0.3275911f, x, 1.0f));
  float q = fmaf(t, 0.5307027145f, -0.7265760135f);
  q = fmaf(t, q, 0.7107068705f);
  q = fmaf(t, q, -0.142248368f);
  q = fmaf(t, q, 0.127414796f);
  const float e = __builtin_amdgcn_exp2f((x * -1.44269504088896340736f) * x);
  const float h = (q * t) * e;
  return PhiExp{u < 0.0f ? h : 1.0f - h, e};
}

// GeLU(u) = u Phi(u) and GeLU'(u) = Phi(u) + u phi(u), phi(u) = exp(-u^2/2) / sqrt(2 pi),
// from phi_as7126: for results rounded to bf16.
__device__ __forceinline__ float gelu_bf16out(float u) {
  return u * phi_as7126(u).phi;
}
__device__ __forceinline__ float gelu_prime_bf16out(float u) {
  const PhiExp p = phi_as7126(u);
  return fmaf(u * 0.39894228040143267794f, p.e, p.phi);
}

}  // namespace tps
