// dequantize.hip -- bf16 reconstruction of MXFP8 / NVFP4 operands for the
// dequantized-backward mode ("Towards Blackwell-Native 8-bit and 4-bit RL",
// High-precision and dequantized backward: the backward GEMMs read the BF16
// dequantization of the exact forward operands).
//
// Each lane decodes 16 consecutive elements (one 16-byte read of MXFP8
// codes, or 8 bytes of packed E2M1) and writes 32 contiguous bytes of bf16.
// Each output is the exact decoded value rounded once to bf16.
#include "pqm_device.hpp"
#include "pqm_internal.hpp"

namespace pqm {

__global__ __launch_bounds__(256) void k_dequant_mxfp8(
    const uint8_t *__restrict__ q, const uint8_t *__restrict__ s, int64_t R, int64_t C,
    uint16_t *__restrict__ y) {
  const int64_t per_row = C / 16;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= R * per_row) return;
  const int64_t row = i / per_row, c = (i % per_row) * 16;
  const uint4 v = *reinterpret_cast<const uint4 *>(q + row * C + c);
  const float sc = e8m0_value(s[row * (C / 32) + c / 32]);
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  uint32_t o[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const uint32_t b0 = (w[k >> 1] >> (16 * (k & 1))) & 0xFFu;
    const uint32_t b1 = (w[k >> 1] >> (16 * (k & 1) + 8)) & 0xFFu;
    // E4M3 value (<= 4 significant bits) times 2^(s-127): exact in binary32
    // unless it overflows, which becomes inf exactly as bf16 rounding would
    const float f0 = e4m3_value(b0 & 0x7F) * sc;
    const float f1 = e4m3_value(b1 & 0x7F) * sc;
    const uint32_t h0 = f32_to_bf16_rne(f0) | ((b0 & 0x80u) << 8);
    const uint32_t h1 = f32_to_bf16_rne(f1) | ((b1 & 0x80u) << 8);
    o[k] = h0 | (h1 << 16);
  }
  uint4 *dst = reinterpret_cast<uint4 *>(y + row * C + c);
  dst[0] = make_uint4(o[0], o[1], o[2], o[3]);
  dst[1] = make_uint4(o[4], o[5], o[6], o[7]);
}

__global__ __launch_bounds__(256) void k_dequant_nvfp4(
    const uint8_t *__restrict__ q, const uint8_t *__restrict__ sb,
    const float *__restrict__ sg, int64_t R, int64_t C, int64_t rows_per_scale,
    uint16_t *__restrict__ y) {
  const int64_t per_row = C / 16;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= R * per_row) return;
  const int64_t row = i / per_row, blk = i % per_row;
  const uint2 v = *reinterpret_cast<const uint2 *>(q + row * (C / 2) + blk * 8);
  const float s_b = e4m3_value(sb[row * per_row + blk] & 0x7F);
  const double s_g = (double)sg[row / rows_per_scale];
  const uint32_t w[2] = {v.x, v.y};
  uint32_t o[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const uint32_t byte = (w[k >> 2] >> (8 * (k & 3))) & 0xFFu;
    uint32_t h[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const uint32_t nib = (byte >> (4 * j)) & 0xFu;
      // q * s_b has at most 6 significant bits (exact in binary32); times
      // s_g it has at most 30, exact in binary64, then one rounding to bf16
      const double v64 = (double)(e2m1_value(nib & 7u) * s_b) * s_g;
      h[j] = f64_to_bf16_rne(v64) | ((nib & 8u) << 12);
    }
    o[k] = h[0] | (h[1] << 16);
  }
  uint4 *dst = reinterpret_cast<uint4 *>(y + row * C + blk * 16);
  dst[0] = make_uint4(o[0], o[1], o[2], o[3]);
  dst[1] = make_uint4(o[4], o[5], o[6], o[7]);
}

hipError_t launch_dequantize(int fmt, const uint8_t *q, const uint8_t *s, const float *sg,
                             int64_t R, int64_t C, int64_t rows_per_scale, uint16_t *y,
                             hipStream_t st) {
  const int64_t n = R * (C / 16);
  if (n == 0) return hipSuccess;
  const unsigned grid = (unsigned)((n + 255) / 256);
  if (fmt == 1)
    hipLaunchKernelGGL(k_dequant_mxfp8, dim3(grid), dim3(256), 0, st, q, s, R, C, y);
  else
    hipLaunchKernelGGL(k_dequant_nvfp4, dim3(grid), dim3(256), 0, st, q, s, sg, R, C,
                       rows_per_scale, y);
  return hipGetLastError();
}

}  // namespace pqm
