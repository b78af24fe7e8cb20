// pqm_device.hpp -- device-side encodings shared by the HIP kernels.
//
// Every function here takes its rounding decision exactly (no fast math, no
// approximate reciprocal).  Formats, from "Towards Blackwell-Native 8-bit
// and 4-bit RL", Format background:
//   E4M3  1 sign, 4 exponent (bias 7), 3 mantissa bits; max 448 = 0x7E;
//         0x7F is NaN and never produced.
//   E8M0  power-of-two scale 2^(b - 127).
//   E2M1  1 sign, 2 exponent, 1 mantissa bit: 0, .5, 1, 1.5, 2, 3, 4, 6.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pqm {

__device__ __forceinline__ float bf16_lo_f32(uint32_t w) {
  return __uint_as_float(w << 16);
}
__device__ __forceinline__ float bf16_hi_f32(uint32_t w) {
  return __uint_as_float(w & 0xFFFF0000u);
}

// Two binary32 values rounded to a bf16 pair (first in the low half) by the
// hardware conversion: nearest even, as f32_to_bf16_rne, for finite values
// and infinities.
__device__ __forceinline__ uint32_t pk_bf16_rne(float lo, float hi) {
  typedef __bf16 pqm_bf2 __attribute__((ext_vector_type(2)));
  const pqm_bf2 v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

// The weighted SwiGLU value silu(g) u p, silu(g) = g / (1 + e^-g), with the
// hardware exponential and reciprocal (about 1 ulp each): the activation of
// every kernel that computes it, so that the fused and the separate passes
// produce the same bits.  For g <= -64, e^-g would overflow binary32 (and e^g
// leave its normal range), so there silu(g) u p = (g u p) e^g is formed with
// e^g = 2^(g log2(e) + 64) 2^-64: both factors stay normal down to g = -131,
// where the true value is far below the smallest bf16 subnormal.
__device__ __forceinline__ float swiglu_f32(float g, float u, float p) {
  if (g > -64.0f) return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)) * u * p;
  const float t = __builtin_amdgcn_exp2f(g * 1.44269504088896341f + 64.0f);
  return ((g * u * p) * t) * 0x1p-64f;
}

// Round a binary32 value to bf16 bits, nearest even (finite or inf input).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// Round an exact binary64 value once to bf16 bits, nearest even; beyond the
// bf16 range -> +-inf.  Used where the exact value has more than 24
// significant bits, so that no intermediate binary32 rounding occurs.
__device__ __forceinline__ uint32_t f64_to_bf16_rne(double v) {
  uint64_t u = (uint64_t)__double_as_longlong(v);
  uint32_t sign = (uint32_t)(u >> 48) & 0x8000u;
  uint64_t a = u & 0x7FFFFFFFFFFFFFFFull;
  int e = (int)(a >> 52) - 1023;
  if (a == 0) return sign;
  if (e >= -126) {
    a += (1ull << 44) - 1ull + ((a >> 45) & 1ull);
    int e2 = (int)(a >> 52) - 1023;
    if (e2 > 127) return sign | 0x7F80u;
    return sign | ((uint32_t)(e2 + 127) << 7) | (uint32_t)((a >> 45) & 0x7Full);
  }
  // bf16 subnormal range: quantum 2^-133; v * 2^133 is an exact scaling.
  double n = __builtin_rint(__longlong_as_double((long long)a) * 0x1p133);
  return sign | (uint32_t)n;  // n == 128 is the smallest normal, bits 0x80
}

// Magnitude code (0..126) of the E4M3 value nearest q (q >= 0, binary64),
// saturating at 448.  q is a correctly rounded quotient whose exact value
// is either an E4M3 midpoint exactly or at least 2^-32 (relative) away from
// every midpoint, so rounding the binary64 value decides as the exact one.
__device__ __forceinline__ uint32_t e4m3_code_f64_sat(double q) {
  if (q >= 448.0) return 126u;
  if (q < 0x1p-6) return (uint32_t)__builtin_rint(q * 512.0);
  uint64_t u = (uint64_t)__double_as_longlong(q);
  u += (1ull << 48) - 1ull + ((u >> 49) & 1ull);  // keep 3 mantissa bits
  uint32_t e = (uint32_t)(u >> 52) - 1023u + 7u;
  return (e << 3) | (uint32_t)((u >> 49) & 7ull);
}

// Exact value of an E4M3 magnitude code.
__device__ __forceinline__ float e4m3_value(uint32_t c) {
  uint32_t e = (c >> 3) & 15u, m = c & 7u;
  if (e == 0) return (float)m * 0x1p-9f;
  return __uint_as_float(((e + 120u) << 23) | (m << 20));
}

// Exact value of an E2M1 magnitude code (0..7).
__device__ __forceinline__ float e2m1_value(uint32_t c) {
  if (c < 2u) return (float)c * 0.5f;
  return __uint_as_float((((c >> 1) + 126u) << 23) | ((c & 1u) << 22));
}

// E8M0 byte b -> 2^(b-127) as binary32 (b = 0 gives the subnormal 2^-127).
__device__ __forceinline__ float e8m0_value(uint32_t b) {
  return b == 0 ? 0x1p-127f : __uint_as_float(b << 23);
}

// E8M0 scale byte of a 1x32 MXFP8 block from the bf16 magnitude bits of its
// maximum (amax = (1 + f/128) 2^(E-127)): the smallest e with
// amax <= 448 * 2^e = 1.75 * 2^(8+e) is E - 127 - 8 + [f > 0x60], clamped
// at e = -127; a zero or subnormal maximum gives e = -127.  Returns e + 127.
// With f > 0x60 exactly when f + 0x1F carries into E, this is
// max(0, ((amax_bits + 0x1F) >> 7) - 8); zero and subnormal maxima (E = 0)
// land below 0.
__device__ __forceinline__ uint32_t mx_scale_byte(uint32_t amax_bits) {
  const int b = (int)((amax_bits + 0x1Fu) >> 7) - 8;
  return (uint32_t)max(b, 0);
}

// NVFP4 block: thresholds for the E2M1 decisions.  The element with
// magnitude |x| gets code  sum_j [ |x| >= U_j ]  where U_j is the smallest
// binary32 value that must round above the midpoint t_j * d
// (t = .25 .75 1.25 1.75 2.5 3.5 5 and d = s_b * s_g, the exact product).
// A tie rounds to the even code: up across t_j for odd j, down for even j.
struct E2M1Thresholds {
  float u[7];
};

__device__ __forceinline__ float next_up_pos(float f) {
  return __uint_as_float(__float_as_uint(f) + 1u);
}

__device__ __forceinline__ void e2m1_thresholds(double d, bool zero_scale,
                                                E2M1Thresholds &th) {
  const double t[7] = {0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0};
#pragma unroll
  for (int j = 0; j < 7; ++j) {
    if (zero_scale) {
      th.u[j] = __builtin_inff();
      continue;
    }
    double T = t[j] * d;  // at most 3 + 28 significant bits: exact
    float f = (float)T;   // nearest binary32
    double fd = (double)f;
    float U;
    if (fd == T)
      U = (j & 1) ? f : next_up_pos(f);  // tie up for odd j
    else
      U = (fd > T) ? f : next_up_pos(f);  // smallest binary32 above T
    th.u[j] = U;
  }
}

__device__ __forceinline__ uint32_t e2m1_code(float a, const E2M1Thresholds &th) {
  uint32_t c = 0;
#pragma unroll
  for (int j = 0; j < 7; ++j) c += (a >= th.u[j]) ? 1u : 0u;
  return c;
}

// ---------------------------------------------------------------------
// Hardware conversions, each compared on gfx950 against the exact rules:
//  * v_cvt_scalef32_pk_fp8_bf16 with the scale operand given as the bits
//    b << 23 (b an E8M0 byte 0..254; b = 0 is the pattern of +0.0f) gives the
//    sign-keeping nearest-even E4M3 of x / 2^(b-127) for every bf16 x whose
//    quotient is at most 448 in magnitude -- all 8.85 million such (x, b)
//    cases, so the scale operand acts exactly as an E8M0 exponent, 2^-127
//    included;
//  * v_cvt_scalef32_pk_fp4_f32 with scale 1.0 gives the nearest-even,
//    saturating, sign-keeping E2M1 of every binary32 input.

typedef __bf16 pqm_v2bf __attribute__((ext_vector_type(2)));
typedef short pqm_v2s __attribute__((ext_vector_type(2)));

// Four E4M3 bytes of x / 2^(b-127) for the bf16 pairs w0, w1 (element order
// w0.lo, w0.hi, w1.lo, w1.hi); scale holds the bits b << 23 of an E8M0 byte b.
__device__ __forceinline__ uint32_t cvt4_e4m3_bf16(uint32_t w0, uint32_t w1, float scale) {
  pqm_v2s r = {0, 0};
  r = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(r, __builtin_bit_cast(pqm_v2bf, w0), scale,
                                                 false);
  r = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(r, __builtin_bit_cast(pqm_v2bf, w1), scale,
                                                 true);
  return __builtin_bit_cast(uint32_t, r);
}

// Packed E2M1 nibbles of two binary32 values into byte `sel` of `old`.
template <int SEL>
__device__ __forceinline__ uint32_t cvt2_e2m1(uint32_t old, float a, float b) {
  return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(old, a, b, 1.0f, SEL);
}

typedef unsigned short pqm_us2 __attribute__((ext_vector_type(2)));

// Per-half unsigned maximum of two packed 16-bit pairs.
__device__ __forceinline__ uint32_t pk_max_u16(uint32_t a, uint32_t b) {
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(pqm_us2, a),
                                                                __builtin_bit_cast(pqm_us2, b)));
}

// Wave-wide maximum of a non-negative float (64 lanes).
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

}  // namespace pqm
