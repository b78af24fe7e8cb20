// quantize_nvfp4.hip -- NVFP4 quantization with an online FP32 outer scale
// ("Towards Blackwell-Native 8-bit and 4-bit RL", Format background: NVFP4
// and Recipe 2: per-token activation scaling; "miniTE technical report",
// 2.2 decode x^ = q * s_b * s_g and 5.6 gs = gamax / 2688).
//
// Per-token scope: one wave owns one row.  The row is read once into
// registers with 16-byte loads (one 1x16 block per lane per step), its
// maximum is reduced across the wave, and all three outputs (packed E2M1,
// E4M3 block scales, FP32 token scale) are written from registers.
//
// Group scope (one outer scale for rows_per_scale rows, e.g. an expert's
// fused gate/up weight): a first kernel reduces each group's maximum into a
// device word with atomicMax on the bf16 magnitude bits; the second kernel
// is the per-row kernel reading that word.  Groups are processed in chunks
// of about 64 MB so the second read of a chunk is served from the
// Infinity Cache rather than HBM.
#include "pqm_device.hpp"
#include "pqm_internal.hpp"

namespace pqm {

// Quantize one 1x16 block held as 8 words of bf16 pairs.  Returns 8 bytes
// of packed nibbles (element 2j low) and the E4M3 scale byte in *sbc_out.
//
// s_b: the quotient a_b / (6 s_g) is taken by a correctly rounded binary64
// division, which decides the E4M3 rounding exactly (see e4m3_code_f64_sat).
//
// Elements, fast path: with d = s_b * s_g (exact in binary64) and inv an
// approximation of 1/d within 2^-22 (binary32 reciprocal of d rounded to
// binary32: at most 1.5 ulp), lo = x * inv (1 - 2^-20) and
// hi = x * inv (1 + 2^-20), each rounded to binary32, bracket the exact
// quotient r = x / d strictly (all roundings together stay below 2^-21, half
// the margin).  E2M1 rounding is monotone, so when lo and hi convert to the
// same codes those are the nearest-even E2M1 of r.  They differ only when
// some r lies within 2^-20 of a rounding midpoint (an exact tie among them);
// such a block, a zero scale, or a tiny d is redone on the exact path, which
// compares each |x| with thresholds derived from the exact midpoints t * d.
// The exact path sits behind a wave-uniform branch: it costs nothing unless
// a lane of the wave needs it.
__device__ __forceinline__ uint2 nvfp4_block(const uint32_t w[8], float s_g, uint32_t *sbc_out) {
  uint32_t mm = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) mm = pk_max_u16(mm, w[i] & 0x7FFF7FFFu);
  const uint32_t mb = max(mm & 0xFFFFu, mm >> 16);
  const float ab = __uint_as_float(mb << 16);
  uint32_t sbc = 0;
  if (s_g != 0.0f) sbc = e4m3_code_f64_sat((double)ab / (6.0 * (double)s_g));
  *sbc_out = sbc;
  const double d = (double)e4m3_value(sbc) * (double)s_g;  // <= 28 bits: exact
  const bool fast_ok = sbc != 0 && d >= 0x1p-120 && d <= 0x1p125;
  const float inv = __builtin_amdgcn_rcpf((float)d);
  const float ilo = inv * (1.0f - 0x1p-20f), ihi = inv * (1.0f + 0x1p-20f);
  uint32_t lo[2] = {0, 0}, hi[2] = {0, 0};
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const uint32_t *ww = w + 4 * h;
    lo[h] = cvt2_e2m1<0>(lo[h], bf16_lo_f32(ww[0]) * ilo, bf16_hi_f32(ww[0]) * ilo);
    lo[h] = cvt2_e2m1<1>(lo[h], bf16_lo_f32(ww[1]) * ilo, bf16_hi_f32(ww[1]) * ilo);
    lo[h] = cvt2_e2m1<2>(lo[h], bf16_lo_f32(ww[2]) * ilo, bf16_hi_f32(ww[2]) * ilo);
    lo[h] = cvt2_e2m1<3>(lo[h], bf16_lo_f32(ww[3]) * ilo, bf16_hi_f32(ww[3]) * ilo);
    hi[h] = cvt2_e2m1<0>(hi[h], bf16_lo_f32(ww[0]) * ihi, bf16_hi_f32(ww[0]) * ihi);
    hi[h] = cvt2_e2m1<1>(hi[h], bf16_lo_f32(ww[1]) * ihi, bf16_hi_f32(ww[1]) * ihi);
    hi[h] = cvt2_e2m1<2>(hi[h], bf16_lo_f32(ww[2]) * ihi, bf16_hi_f32(ww[2]) * ihi);
    hi[h] = cvt2_e2m1<3>(hi[h], bf16_lo_f32(ww[3]) * ihi, bf16_hi_f32(ww[3]) * ihi);
  }
  uint2 out = make_uint2(lo[0], lo[1]);
  const bool need = !(fast_ok && lo[0] == hi[0] && lo[1] == hi[1]);
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

// One wave per row, one row per wave (the hardware dispatcher balances the
// rows over the CUs; a persistent loop left a partial last round).  Lane l
// owns the 1x16 blocks l + 64 j (two 16-byte loads each), all issued before
// any use; NB blocks per lane (cols <= 1024 NB).  When amax_ws is non-null
// the outer scale comes from the group word amax_ws[row / rows_per_scale]
// instead of the row.
template <int NB>
__global__ __launch_bounds__(256) void k_quantize_nvfp4_rows(
    const uint16_t *__restrict__ x, int64_t R, int64_t C, int64_t ld,
    int64_t row_begin, int64_t row_end, int64_t rows_per_scale,
    const uint32_t *__restrict__ amax_ws, uint8_t *__restrict__ q,
    uint8_t *__restrict__ sb, float *__restrict__ sg) {
  const int lane = threadIdx.x & 63;
  const int64_t nblk = C / 16;
  const int64_t row = row_begin + (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= row_end) return;  // whole wave exits together
  const uint16_t *xr = x + row * ld;
  uint32_t w[NB][8];
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    const int64_t blk = lane + 64 * b;
    uint4 v0 = make_uint4(0, 0, 0, 0), v1 = v0;
    if (blk < nblk) {
      v0 = *reinterpret_cast<const uint4 *>(xr + blk * 16);
      v1 = *reinterpret_cast<const uint4 *>(xr + blk * 16 + 8);
    }
    w[b][0] = v0.x; w[b][1] = v0.y; w[b][2] = v0.z; w[b][3] = v0.w;
    w[b][4] = v1.x; w[b][5] = v1.y; w[b][6] = v1.z; w[b][7] = v1.w;
  }
  float A;
  if (amax_ws) {
    A = __uint_as_float(amax_ws[row / rows_per_scale] << 16);
  } else {
    uint32_t m = 0;
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int i = 0; i < 8; ++i) m = pk_max_u16(m, w[b][i] & 0x7FFF7FFFu);
    m = max(m & 0xFFFFu, m >> 16);
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, o, 64));
    A = __uint_as_float(m << 16);
  }
  const float s_g = __fdiv_rn(A, 2688.0f);  // one correctly rounded division
  if (lane == 0 && (amax_ws == nullptr || row % rows_per_scale == 0))
    sg[row / rows_per_scale] = s_g;
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    if ((int64_t)64 * b < nblk) {  // uniform: the exact path's ballot needs the wave
      const int64_t blk = lane + 64 * b;
      uint32_t code;
      const uint2 packed = nvfp4_block(w[b], s_g, &code);
      if (blk < nblk) {
        *reinterpret_cast<uint2 *>(q + row * (C / 2) + blk * 8) = packed;
        sb[row * nblk + blk] = (uint8_t)code;
      }
    }
  }
}

// Group maximum: each workgroup reduces rows_per_wg rows of one group (wave
// w takes rows w, w+4, ...; 16-byte loads, packed 16-bit max) and folds the
// result into amax_ws[group] with one atomicMax (bf16 magnitude bits:
// integer order equals value order for non-negative finite values).
template <int NB>
__global__ __launch_bounds__(256) void k_group_amax(
    const uint16_t *__restrict__ x, int64_t C, int64_t ld, int64_t row_begin,
    int64_t row_end, int64_t rows_per_scale, int64_t rows_per_wg,
    uint32_t *__restrict__ amax_ws) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t nblk = C / 16;
  const int64_t r0 = row_begin + (int64_t)blockIdx.x * rows_per_wg;
  int64_t r1 = r0 + rows_per_wg;
  if (r1 > row_end) r1 = row_end;
  uint32_t m = 0;
#pragma unroll 4
  for (int64_t r = r0 + wave; r < r1; r += 4) {
    const uint16_t *xr = x + r * ld;
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const int64_t blk = lane + 64 * b;
      if (blk < nblk) {
        const uint4 v0 = *reinterpret_cast<const uint4 *>(xr + blk * 16);
        const uint4 v1 = *reinterpret_cast<const uint4 *>(xr + blk * 16 + 8);
        m = pk_max_u16(m, pk_max_u16(pk_max_u16(v0.x & 0x7FFF7FFFu, v0.y & 0x7FFF7FFFu),
                                     pk_max_u16(v0.z & 0x7FFF7FFFu, v0.w & 0x7FFF7FFFu)));
        m = pk_max_u16(m, pk_max_u16(pk_max_u16(v1.x & 0x7FFF7FFFu, v1.y & 0x7FFF7FFFu),
                                     pk_max_u16(v1.z & 0x7FFF7FFFu, v1.w & 0x7FFF7FFFu)));
      }
    }
  }
  m = max(m & 0xFFFFu, m >> 16);
  __shared__ uint32_t red[4];
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, o, 64));
  if (lane == 0) red[wave] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    m = max(max(red[0], red[1]), max(red[2], red[3]));
    atomicMax(&amax_ws[r0 / rows_per_scale], m);
  }
}

__global__ void k_fill_u32(uint32_t *p, int64_t n, uint32_t v) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

template <int NB>
static void launch_rows(const uint16_t *x, int64_t R, int64_t C, int64_t ld, int64_t rb,
                        int64_t re, int64_t rps, const uint32_t *ws, uint8_t *q,
                        uint8_t *sb, float *sg, hipStream_t st) {
  const unsigned grid = (unsigned)((re - rb + 3) / 4);
  hipLaunchKernelGGL((k_quantize_nvfp4_rows<NB>), dim3(grid), dim3(256), 0, st, x, R, C, ld,
                     rb, re, rps, ws, q, sb, sg);
}

static void dispatch_rows(const uint16_t *x, int64_t R, int64_t C, int64_t ld, int64_t rb,
                          int64_t re, int64_t rps, const uint32_t *ws, uint8_t *q,
                          uint8_t *sb, float *sg, hipStream_t st) {
  const int64_t per_lane = (C / 16 + 63) / 64;
  if (per_lane <= 1) launch_rows<1>(x, R, C, ld, rb, re, rps, ws, q, sb, sg, st);
  else if (per_lane <= 2) launch_rows<2>(x, R, C, ld, rb, re, rps, ws, q, sb, sg, st);
  else if (per_lane <= 4) launch_rows<4>(x, R, C, ld, rb, re, rps, ws, q, sb, sg, st);
  else if (per_lane <= 8) launch_rows<8>(x, R, C, ld, rb, re, rps, ws, q, sb, sg, st);
  else launch_rows<16>(x, R, C, ld, rb, re, rps, ws, q, sb, sg, st);
}

int64_t nvfp4_max_cols() { return 16 * 1024; }

size_t nvfp4_workspace_bytes(int64_t R, int64_t rows_per_scale) {
  if (rows_per_scale <= 1 || R == 0) return 0;
  return (size_t)(R / rows_per_scale) * sizeof(uint32_t);
}

hipError_t launch_quantize_nvfp4(const uint16_t *x, int64_t R, int64_t C, int64_t ld,
                                 int64_t rows_per_scale, uint8_t *q, uint8_t *sb, float *sg,
                                 void *workspace, hipStream_t st) {
  if (R == 0 || C == 0) return hipSuccess;
  if (rows_per_scale == 1) {
    dispatch_rows(x, R, C, ld, 0, R, 1, nullptr, q, sb, sg, st);
    return hipGetLastError();
  }
  uint32_t *ws = static_cast<uint32_t *>(workspace);
  const int64_t G = R / rows_per_scale;
  hipLaunchKernelGGL(k_fill_u32, dim3((unsigned)((G + 255) / 256)), dim3(256), 0, st, ws, G, 0u);
  const int64_t group_bytes = rows_per_scale * C * 2;
  int64_t groups_per_chunk = ((int64_t)64 << 20) / (group_bytes > 0 ? group_bytes : 1);
  if (groups_per_chunk < 1) groups_per_chunk = 1;
  // rows per amax workgroup: about 64 KB of input each, within one group
  int64_t rpw = (65536 / (C * 2));
  if (rpw < 1) rpw = 1;
  while (rows_per_scale % rpw) --rpw;
  const int64_t per_lane = (C / 16 + 63) / 64;
  for (int64_t g0 = 0; g0 < G; g0 += groups_per_chunk) {
    const int64_t g1 = (g0 + groups_per_chunk < G) ? g0 + groups_per_chunk : G;
    const int64_t rb = g0 * rows_per_scale, re = g1 * rows_per_scale;
    const dim3 ga((unsigned)((re - rb) / rpw));
    if (per_lane <= 1)
      hipLaunchKernelGGL(k_group_amax<1>, ga, dim3(256), 0, st, x, C, ld, rb, re, rows_per_scale, rpw, ws);
    else if (per_lane <= 2)
      hipLaunchKernelGGL(k_group_amax<2>, ga, dim3(256), 0, st, x, C, ld, rb, re, rows_per_scale, rpw, ws);
    else if (per_lane <= 4)
      hipLaunchKernelGGL(k_group_amax<4>, ga, dim3(256), 0, st, x, C, ld, rb, re, rows_per_scale, rpw, ws);
    else if (per_lane <= 8)
      hipLaunchKernelGGL(k_group_amax<8>, ga, dim3(256), 0, st, x, C, ld, rb, re, rows_per_scale, rpw, ws);
    else
      hipLaunchKernelGGL(k_group_amax<16>, ga, dim3(256), 0, st, x, C, ld, rb, re, rows_per_scale, rpw, ws);
    dispatch_rows(x, R, C, ld, rb, re, rows_per_scale, ws, q, sb, sg, st);
  }
  return hipGetLastError();
}

}  // namespace pqm
