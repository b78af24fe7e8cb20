// nvfp4_encode.hpp -- the NVFP4 encoding of 1x16 bf16 blocks under a given
// binary32 outer scale s_g = A / 2688 ("Towards Blackwell-Native 8-bit and
// 4-bit RL", Format background: NVFP4; "miniTE technical report", 2.2 and
// 5.6): E4M3 block scale nearest to a_b / (6 s_g), E2M1 codes nearest to
// x / (s_b s_g), both decided exactly.  Shared by the quantizers and by the
// FC2 kernel that encodes its operand under a running row maximum.
#pragma once
#include "pqm_device.hpp"

namespace pqm {

// Row constants of the NVFP4 encoding.  The quantizers give a wave one row,
// so these are wave-uniform there; nvfp4_block is also exact when the lanes of
// a wave hold blocks of different rows (the whole wave still calls it, for
// its exact-path ballot).
struct Nvfp4Row {
  float s_g;    // outer scale A / 2688, one correctly rounded division
  float inv6;   // 1 / (6 s_g) rounded to binary32 (within 2^-24)
  int dir;      // sign of A - 2688 s_g: +1, -1, or 0 when s_g is exact
  bool fast;    // s_g normal and small enough for the bracketed paths
};

__device__ __forceinline__ Nvfp4Row nvfp4_row(float A) {
  Nvfp4Row r;
  r.s_g = __fdiv_rn(A, 2688.0f);
  const float res = __builtin_fmaf(-2688.0f, r.s_g, A);  // exact sign of A - 2688 s_g
  r.dir = res > 0.0f ? 1 : (res < 0.0f ? -1 : 0);
  // s_g >= 2^-90 keeps d = s_b s_g >= 2^-99, so that d's trailing binary32
  // part is normal; s_g <= 2^116 keeps d and 1/d normal
  r.fast = r.s_g >= 0x1p-90f && r.s_g <= 0x1p116f;
  r.inv6 = r.fast ? (float)(1.0 / (6.0 * (double)r.s_g)) : 0.0f;
  return r;
}

// Magnitude code (0..126) of the E4M3 value nearest v >= 0 (binary32),
// ties to even, saturating at 448.
__device__ __forceinline__ uint32_t e4m3_code_f32_sat(float v) {
  uint32_t c;
  if (v < 0x1p-6f) {
    c = (uint32_t)__builtin_rintf(v * 512.0f);  // subnormal quantum 2^-9: exact scaling
  } else {
    uint32_t u = __float_as_uint(v);
    u += 0x7FFFFu + ((u >> 20) & 1u);  // keep 3 mantissa bits, nearest even
    c = (((u >> 23) - 120u) << 3) | ((u >> 20) & 7u);
  }
  return min(c, 126u);
}

// Of two codes that differ (or not), the one a near-tie resolves to: the
// quotient the codes were taken from is Q / (1 + eta) with Q the quotient
// computed with A / 2688 in place of s_g and s_g = (A / 2688)(1 + eta).
// dir > 0 (eta < 0): above Q; dir < 0: below; dir == 0: Q itself, a tie
// going to the even code (low bit of the magnitude code clear).
__device__ __forceinline__ uint32_t resolve_code(uint32_t lo, uint32_t hi, int dir) {
  if (dir > 0) return hi;
  if (dir < 0) return lo;
  return (lo & 1u) ? hi : lo;
}

// Quantize one 1x16 block held as 8 words of bf16 pairs.  Returns 8 bytes of
// packed nibbles (element 2j low) and the E4M3 scale code in *sbc_out.
//
// Both roundings are taken from binary32 quotients bracketed tightly enough
// that a disagreement between the two ends can only come from an exact
// rational tie of the ideal quotient, which the row's dir then resolves:
//  * s_b = E4M3(a_b / (6 s_g)): v = a_b * inv6 is within 2^-23 of the exact
//    quotient; v (1 -+ 2^-21) bracket it.  When the two ends round to
//    different codes, a midpoint m lies within 2^-19.9 of a_b / (6 s_g), and
//    so within 2^-19.8 of P = 448 a_b / A.  P - m is a ratio of short
//    integers (448 = 7 * 2^6, 8-bit a_b and A, 5-bit m), so it is either 0
//    or at least 2^-16.8 relative (2^-12.8 by exhaustive search over all
//    significands): P = m exactly, and the true quotient P / (1 + eta) lies
//    on the side dir says.
//  * elements: with d = s_b s_g (exact in binary64) and inv the binary32
//    rounding of 1/d (one Newton step on the binary32 reciprocal of d's
//    leading part, with d's trailing part), x * inv (1 -+ 2^-22) bracket
//    x / d strictly.  A disagreement puts an E2M1 midpoint t within 2^-20.2
//    of x / d, hence within 2^-20.1 of Q = 2688 x / (s_b A); Q - t is either
//    0 or at least 2^-19.38 relative (8-bit x and A, 4-bit s_b, 3-bit odd
//    part of t, 2688 = 21 * 2^7; 2^-13.8 by exhaustive search over all
//    significands and scales), so Q = t and dir decides again.  Where the
//    ends agree, E2M1 rounding being monotone, their code is the exact one.
// Blocks with s_b = 0 (all elements encode to a signed zero) and rows whose
// s_g lies outside the range the bracket arithmetic covers (zero rows
// included; their s_b comes from a correctly rounded binary64 division) take
// the exact threshold path behind a wave-uniform branch.
__device__ __forceinline__ uint2 nvfp4_block(const uint32_t w[8], const Nvfp4Row &row,
                                             uint32_t *sbc_out) {
  uint32_t mm = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) mm = pk_max_u16(mm, w[i] & 0x7FFF7FFFu);
  const uint32_t mb = max(mm & 0xFFFFu, mm >> 16);
  const float ab = __uint_as_float(mb << 16);
  // ---- block scale -------------------------------------------------------
  uint32_t sbc;
  if (row.fast) {
    const float v = ab * row.inv6;
    sbc = resolve_code(e4m3_code_f32_sat(v * (1.0f - 0x1p-21f)),
                       e4m3_code_f32_sat(v * (1.0f + 0x1p-21f)), row.dir);
  } else {
    // correctly rounded binary64 quotient: decides the E4M3 rounding exactly
    // (see e4m3_code_f64_sat); s_g = 0 is a zero row
    sbc = row.s_g != 0.0f ? e4m3_code_f64_sat((double)ab / (6.0 * (double)row.s_g)) : 0u;
  }
  *sbc_out = sbc;
  // ---- elements ----------------------------------------------------------
  const double d = (double)e4m3_value(sbc) * (double)row.s_g;  // <= 28 bits: exact
  const float dh = (float)d;
  const float dl = (float)(d - (double)dh);
  const float i0 = __builtin_amdgcn_rcpf(dh);
  const float e = __builtin_fmaf(-dl, i0, __builtin_fmaf(-dh, i0, 1.0f));
  const float inv = __builtin_fmaf(i0, e, i0);
  uint2 out;
  if (row.dir != 0) {
    const float k = inv * (row.dir > 0 ? 1.0f + 0x1p-22f : 1.0f - 0x1p-22f);
    uint32_t o[2] = {0, 0};
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const uint32_t *ww = w + 4 * h;
      o[h] = cvt2_e2m1<0>(o[h], bf16_lo_f32(ww[0]) * k, bf16_hi_f32(ww[0]) * k);
      o[h] = cvt2_e2m1<1>(o[h], bf16_lo_f32(ww[1]) * k, bf16_hi_f32(ww[1]) * k);
      o[h] = cvt2_e2m1<2>(o[h], bf16_lo_f32(ww[2]) * k, bf16_hi_f32(ww[2]) * k);
      o[h] = cvt2_e2m1<3>(o[h], bf16_lo_f32(ww[3]) * k, bf16_hi_f32(ww[3]) * k);
    }
    out = make_uint2(o[0], o[1]);
  } else {
    const float klo = inv * (1.0f - 0x1p-22f), khi = inv * (1.0f + 0x1p-22f);
    uint32_t lo[2] = {0, 0}, hi[2] = {0, 0};
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const uint32_t *ww = w + 4 * h;
      lo[h] = cvt2_e2m1<0>(lo[h], bf16_lo_f32(ww[0]) * klo, bf16_hi_f32(ww[0]) * klo);
      lo[h] = cvt2_e2m1<1>(lo[h], bf16_lo_f32(ww[1]) * klo, bf16_hi_f32(ww[1]) * klo);
      lo[h] = cvt2_e2m1<2>(lo[h], bf16_lo_f32(ww[2]) * klo, bf16_hi_f32(ww[2]) * klo);
      lo[h] = cvt2_e2m1<3>(lo[h], bf16_lo_f32(ww[3]) * klo, bf16_hi_f32(ww[3]) * klo);
      hi[h] = cvt2_e2m1<0>(hi[h], bf16_lo_f32(ww[0]) * khi, bf16_hi_f32(ww[0]) * khi);
      hi[h] = cvt2_e2m1<1>(hi[h], bf16_lo_f32(ww[1]) * khi, bf16_hi_f32(ww[1]) * khi);
      hi[h] = cvt2_e2m1<2>(hi[h], bf16_lo_f32(ww[2]) * khi, bf16_hi_f32(ww[2]) * khi);
      hi[h] = cvt2_e2m1<3>(hi[h], bf16_lo_f32(ww[3]) * khi, bf16_hi_f32(ww[3]) * khi);
      // exact ties: of two differing nibbles take the one with an even code
      const uint32_t odd = (lo[h] & 0x11111111u) * 0xFu;
      lo[h] = (lo[h] & ~odd) | (hi[h] & odd);
    }
    out = make_uint2(lo[0], lo[1]);
  }
  const bool need = sbc == 0 || !row.fast;
  if (__builtin_amdgcn_ballot_w64(need) != 0) {
    if (need) {  // exact path
      E2M1Thresholds th;
      e2m1_thresholds(d, sbc == 0, th);
      uint32_t o[2] = {0, 0};
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const uint32_t a = w[i] & 0xFFFFu, b = w[i] >> 16;
        const uint32_t n0 = e2m1_code(__uint_as_float((a & 0x7FFFu) << 16), th) | ((a >> 12) & 8u);
        const uint32_t n1 = e2m1_code(__uint_as_float((b & 0x7FFFu) << 16), th) | ((b >> 12) & 8u);
        o[i >> 2] |= (n0 | (n1 << 4)) << (8 * (i & 3));
      }
      out = make_uint2(o[0], o[1]);
    }
  }
  return out;
}

}  // namespace pqm
