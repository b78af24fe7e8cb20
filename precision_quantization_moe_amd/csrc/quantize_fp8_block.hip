// quantize_fp8_block.hip -- DeepSeek-V3-style block-scaled FP8 ("Towards
// Blackwell-Native 8-bit and 4-bit RL", Why Blackwell-native recipes: 128 x 128
// weight blocks and 1 x 128 activation tiles, each with an FP32 scale computed
// online; "PR #2396 report", Choose a precision: FP8 block-wise, 128 x 128,
// FP32 scales).
//
// For a block with absolute maximum A: s = A / 448 rounded once to binary32,
// q = nearest E4M3 to the exact quotient x / s, ties to even, saturating at
// 448; A = 0 gives s = 0 and signed zeros.
//
// Exactness: v = x / s is the IEEE (correctly rounded) binary32 quotient.
// Every E4M3 midpoint m has at most 5 significant bits, so it is a binary32
// value; if m lay strictly between x / s and v, m would be a closer binary32
// value than v.  So v and x / s are on the same side of every midpoint
// unless v is a midpoint itself, and only then is the side taken from the
// sign of |x| - m s, which binary64 holds exactly (m s has at most 29
// significant bits and lies within a factor 2 of |x|).
#include "pqm_device.hpp"
#include "pqm_internal.hpp"
#include "pqmoe.h"

namespace pqm {

// Is a (> 0, <= 448) the midpoint of two adjacent E4M3 values?  Normal
// E4M3 values are 8 significand steps per binade: a midpoint has its fourth
// fraction bit set and none below.  Below 2^-6 the step is 2^-9: a midpoint
// is an odd multiple of 2^-10.
__device__ __forceinline__ bool e4m3_midpoint(float a) {
  if (a >= 0x1p-6f) return (__float_as_uint(a) & 0xFFFFFu) == 0x80000u;
  const float t = a * 1024.0f;  // exact
  return t == truncf(t) && (((int)t) & 1);
}

// A binary32 value whose nearest-even E4M3 is that of the exact x / s
// (s > 0): the IEEE quotient, clamped to +-448, moved one ulp off an E4M3
// midpoint toward x / s when it landed on one and x / s is not that midpoint.
__device__ __forceinline__ float e4m3_operand(float x, float s) {
  float v = __fdiv_rn(x, s);
  v = fminf(fmaxf(v, -448.0f), 448.0f);  // |x / s| <= 448 (1 + 2^-24): nearest is 448
  const float a = fabsf(v);
  if (e4m3_midpoint(a)) {
    const double r = fabs((double)x) - (double)a * (double)s;
    if (r != 0.0)
      v = copysignf(__uint_as_float(__float_as_uint(a) + (r > 0.0 ? 1u : 0xFFFFFFFFu)), v);
  }
  return v;
}

// Four E4M3 bytes of the bf16 pair words w0, w1 (element order w0.lo, w0.hi,
// w1.lo, w1.hi) for scale s; s == 0 gives signed zeros.
__device__ __forceinline__ uint32_t fp8b_word(uint32_t w0, uint32_t w1, float s) {
  if (s == 0.0f)
    return ((w0 >> 8) & 0x80u) | ((w0 >> 16) & 0x8000u) | ((w1 << 8) & 0x800000u) |
           (w1 & 0x80000000u);
  int r = __builtin_amdgcn_cvt_pk_fp8_f32(e4m3_operand(bf16_lo_f32(w0), s),
                                          e4m3_operand(bf16_hi_f32(w0), s), 0, false);
  r = __builtin_amdgcn_cvt_pk_fp8_f32(e4m3_operand(bf16_lo_f32(w1), s),
                                      e4m3_operand(bf16_hi_f32(w1), s), r, true);
  return (uint32_t)r;
}

__device__ __forceinline__ float abs_max8(const uint4 &v) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  float m = 0.0f;
#pragma unroll
  for (int k = 0; k < 4; ++k)
    m = fmaxf(m, fmaxf(fabsf(bf16_lo_f32(w[k])), fabsf(bf16_hi_f32(w[k]))));
  return m;
}

// 1 x 128 tiles: one wave per (row, 512 columns); lane l takes 8 elements
// (16 bytes) at column 8 l, so 16 lanes hold one tile.
__global__ __launch_bounds__(256) void k_quantize_fp8_tiles(const uint16_t *__restrict__ x,
                                                            int64_t R, int64_t C, int64_t ld,
                                                            int64_t chunks,
                                                            uint8_t *__restrict__ q,
                                                            float *__restrict__ s) {
  const int lane = threadIdx.x & 63;
  const int64_t w = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (w >= R * chunks) return;
  const int64_t row = w / chunks, c0 = (w % chunks) * 512 + 8 * lane;
  const bool in = c0 < C;  // C % 128 == 0: a tile is all in or all out
  uint4 v = make_uint4(0, 0, 0, 0);
  if (in) v = *reinterpret_cast<const uint4 *>(x + row * ld + c0);
  float a = abs_max8(v);
#pragma unroll
  for (int o = 8; o >= 1; o >>= 1) a = fmaxf(a, __shfl_xor(a, o, 64));
  if (!in) return;
  const float sc = __fdiv_rn(a, 448.0f);
  if ((lane & 15) == 0) s[row * (C / 128) + c0 / 128] = sc;
  *reinterpret_cast<uint2 *>(q + row * C + c0) = make_uint2(fp8b_word(v.x, v.y, sc),
                                                            fp8b_word(v.z, v.w, sc));
}

// 128 x 128 blocks: one workgroup per block; thread t takes 8 elements of
// rows t / 16 + 16 i (i = 0..7) at column 8 (t % 16).
__global__ __launch_bounds__(256) void k_quantize_fp8_blocks(const uint16_t *__restrict__ x,
                                                             int64_t C, int64_t ld,
                                                             uint8_t *__restrict__ q,
                                                             float *__restrict__ s) {
  __shared__ float part[4];
  const int64_t CB = C / 128;
  const int64_t rb = blockIdx.x / CB, cb = blockIdx.x % CB;
  const int t = threadIdx.x;
  const int64_t r0 = rb * 128 + t / 16, c0 = cb * 128 + 8 * (t % 16);
  uint4 v[8];
  float a = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    v[i] = *reinterpret_cast<const uint4 *>(x + (r0 + 16 * i) * ld + c0);
    a = fmaxf(a, abs_max8(v[i]));
  }
  a = wave_max(a);
  if ((t & 63) == 0) part[t >> 6] = a;
  __syncthreads();
  a = fmaxf(fmaxf(part[0], part[1]), fmaxf(part[2], part[3]));
  const float sc = __fdiv_rn(a, 448.0f);
  if (t == 0) s[blockIdx.x] = sc;
#pragma unroll
  for (int i = 0; i < 8; ++i)
    *reinterpret_cast<uint2 *>(q + (r0 + 16 * i) * C + c0) =
        make_uint2(fp8b_word(v[i].x, v[i].y, sc), fp8b_word(v[i].z, v[i].w, sc));
}

hipError_t launch_quantize_fp8_block(const uint16_t *x, int64_t R, int64_t C, int64_t ld,
                                     int64_t br, uint8_t *q, float *s, hipStream_t st) {
  if (R == 0 || C == 0) return hipSuccess;
  if (br == 1) {
    const int64_t chunks = (C + 511) / 512, waves = R * chunks;
    hipLaunchKernelGGL(k_quantize_fp8_tiles, dim3((unsigned)((waves + 3) / 4)), dim3(256), 0, st,
                       x, R, C, ld, chunks, q, s);
  } else {
    hipLaunchKernelGGL(k_quantize_fp8_blocks, dim3((unsigned)((R / 128) * (C / 128))), dim3(256),
                       0, st, x, C, ld, q, s);
  }
  return hipGetLastError();
}

}  // namespace pqm
