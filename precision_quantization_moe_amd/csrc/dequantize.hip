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

// 16 bf16 outputs (32 bytes) with streaming stores: written once, not re-read
// (measured 8 % faster for the NVFP4 reconstruction, neutral for MXFP8).
__device__ __forceinline__ void store_out(uint16_t *y, const uint32_t (&o)[8]) {
  typedef uint32_t u4v __attribute__((ext_vector_type(4)));
  __builtin_nontemporal_store(u4v{o[0], o[1], o[2], o[3]}, reinterpret_cast<u4v *>(y));
  __builtin_nontemporal_store(u4v{o[4], o[5], o[6], o[7]}, reinterpret_cast<u4v *>(y) + 1);
}

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

// bf16 bits of the 8 magnitudes v * d, v in {0, .5, 1, 1.5, 2, 3, 4, 6}, for
// d = s_b s_g > 0 exact in binary64, as byte tables for v_perm_b32 (lo0 /
// lo1: low bytes of entries 0-3 / 4-7, hi0 / hi1: high bytes).  When d and
// 6 d lie in the normal bf16 range, 2^k d rounds to 2^k bf16(d), so two
// roundings (of d and of 1.5 d) give all eight entries; otherwise each
// entry is rounded on its own.
struct Nv4Lut {
  uint32_t lo0, lo1, hi0, hi1;
};

__device__ __forceinline__ uint32_t bf16_normal_rne(double v) {  // v > 0, normal in bf16
  uint64_t a = (uint64_t)__double_as_longlong(v);
  a += (1ull << 44) - 1ull + ((a >> 45) & 1ull);
  return (uint32_t)((((a >> 52) - 1023 + 127) << 7) | ((a >> 45) & 0x7Full));
}

__device__ __forceinline__ Nv4Lut nv4_lut(double d) {
  uint32_t t[8];
  const int e = (int)(((uint64_t)__double_as_longlong(d) >> 52) & 0x7FF) - 1023;
  if (d > 0.0 && e >= -125 && e <= 124) {
    const uint32_t r1 = bf16_normal_rne(d), r3 = bf16_normal_rne(1.5 * d);
    t[0] = 0;
    t[1] = r1 - 0x80u;
    t[2] = r1;
    t[3] = r3;
    t[4] = r1 + 0x80u;
    t[5] = r3 + 0x80u;
    t[6] = r1 + 0x100u;
    t[7] = r3 + 0x100u;
  } else {
#pragma unroll
    for (int k = 0; k < 8; ++k) t[k] = f64_to_bf16_rne((double)e2m1_value((uint32_t)k) * d);
  }
  Nv4Lut L;
  L.lo0 = (t[0] & 0xFF) | ((t[1] & 0xFF) << 8) | ((t[2] & 0xFF) << 16) | (t[3] << 24);
  L.lo1 = (t[4] & 0xFF) | ((t[5] & 0xFF) << 8) | ((t[6] & 0xFF) << 16) | (t[7] << 24);
  L.hi0 = (t[0] >> 8) | ((t[1] >> 8) << 8) | ((t[2] >> 8) << 16) | ((t[3] >> 8) << 24);
  L.hi1 = (t[4] >> 8) | ((t[5] >> 8) << 8) | ((t[6] >> 8) << 16) | ((t[7] >> 8) << 24);
  return L;
}

// 8 packed E2M1 (element 2j in the low nibble of byte j) -> 8 bf16 in o[4].
__device__ __forceinline__ void nv4_word(uint32_t w, const Nv4Lut &L, uint32_t *o) {
  const uint32_t ie = w & 0x07070707u, io = (w >> 4) & 0x07070707u;
  const uint32_t le = __builtin_amdgcn_perm(L.lo1, L.lo0, ie), he = __builtin_amdgcn_perm(L.hi1, L.hi0, ie);
  const uint32_t lo = __builtin_amdgcn_perm(L.lo1, L.lo0, io), ho = __builtin_amdgcn_perm(L.hi1, L.hi0, io);
  const uint32_t e02 = __builtin_amdgcn_perm(he, le, 0x05010400u);  // elements 0, 2
  const uint32_t e46 = __builtin_amdgcn_perm(he, le, 0x07030602u);  // 4, 6
  const uint32_t o13 = __builtin_amdgcn_perm(ho, lo, 0x05010400u);  // 1, 3
  const uint32_t o57 = __builtin_amdgcn_perm(ho, lo, 0x07030602u);  // 5, 7
  // sign of element 2j: bit 3 of byte j; of element 2j+1: bit 7
  const uint32_t se = (w << 4) & 0x80808080u, so = w & 0x80808080u;
  o[0] = __builtin_amdgcn_perm(o13, e02, 0x05040100u) | __builtin_amdgcn_perm(so, se, 0x040C000Cu);
  o[1] = __builtin_amdgcn_perm(o13, e02, 0x07060302u) | __builtin_amdgcn_perm(so, se, 0x050C010Cu);
  o[2] = __builtin_amdgcn_perm(o57, e46, 0x05040100u) | __builtin_amdgcn_perm(so, se, 0x060C020Cu);
  o[3] = __builtin_amdgcn_perm(o57, e46, 0x07060302u) | __builtin_amdgcn_perm(so, se, 0x070C030Cu);
}

// Lane i decodes the 16-element block i of the flattened tensor (blocks
// are contiguous across rows): 8 bytes of q, one scale byte, 32 bytes out.
// Its outer scale is that of group i / blocks_per_group.
__global__ __launch_bounds__(256) void k_dequant_nvfp4(
    const uint8_t *__restrict__ q, const uint8_t *__restrict__ sb,
    const float *__restrict__ sg, int64_t nblk, int64_t blocks_per_group,
    uint16_t *__restrict__ y) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= nblk) return;
  const uint2 v = *reinterpret_cast<const uint2 *>(q + i * 8);
  // group = floor(i / blocks_per_group): binary64 quotient, then corrected
  int64_t grp = (int64_t)((double)i / (double)blocks_per_group);
  if (grp * blocks_per_group > i) --grp;
  if ((grp + 1) * blocks_per_group <= i) ++grp;
  // s_b s_g: <= 4 + 24 significant bits, exact in binary64; each output is
  // q s_b s_g rounded once to bf16
  const double d = (double)e4m3_value(sb[i] & 0x7Fu) * (double)sg[grp];
  const Nv4Lut L = nv4_lut(d);
  uint32_t o[8];
  nv4_word(v.x, L, o);
  nv4_word(v.y, L, o + 4);
  store_out(y + i * 16, o);
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
    hipLaunchKernelGGL(k_dequant_nvfp4, dim3(grid), dim3(256), 0, st, q, s, sg, n,
                       (C / 16) * rows_per_scale, y);
  return hipGetLastError();
}

}  // namespace pqm
