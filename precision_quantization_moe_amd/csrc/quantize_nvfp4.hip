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

// Quantize one 1x16 block held as 8 words of bf16 pairs.  Writes 8 bytes of
// packed nibbles (element 2j low) and returns the E4M3 scale byte.
__device__ __forceinline__ uint32_t nvfp4_block(const uint32_t w[8], float s_g,
                                                uint2 &packed) {
  uint32_t mb = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    mb = max(mb, w[i] & 0x7FFFu);
    mb = max(mb, (w[i] >> 16) & 0x7FFFu);
  }
  const float ab = __uint_as_float(mb << 16);
  uint32_t sbc = 0;
  if (s_g != 0.0f) {
    // exact quotient decided in binary64 (correctly rounded division)
    const double qd = (double)ab / (6.0 * (double)s_g);
    sbc = e4m3_code_f64_sat(qd);
  }
  E2M1Thresholds th;
  e2m1_thresholds((double)e4m3_value(sbc) * (double)s_g, sbc == 0, th);
  uint32_t out[2] = {0, 0};
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t lo = w[i] & 0xFFFFu, hi = w[i] >> 16;
    const uint32_t n0 = e2m1_code(__uint_as_float((lo & 0x7FFFu) << 16), th) | ((lo >> 12) & 8u);
    const uint32_t n1 = e2m1_code(__uint_as_float((hi & 0x7FFFu) << 16), th) | ((hi >> 12) & 8u);
    out[i >> 2] |= (n0 | (n1 << 4)) << (8 * (i & 3));
  }
  packed = make_uint2(out[0], out[1]);
  return sbc;
}

// Rows are processed one per wave.  NB = blocks per lane held in registers
// (cols <= NB * 16 * 64).  When amax_ws is non-null the outer scale comes
// from the group word amax_ws[row / rows_per_scale] instead of the row.
template <int NB>
__global__ __launch_bounds__(256) void k_quantize_nvfp4_rows(
    const uint16_t *__restrict__ x, int64_t R, int64_t C, int64_t ld,
    int64_t row_begin, int64_t row_end, int64_t rows_per_scale,
    const uint32_t *__restrict__ amax_ws, uint8_t *__restrict__ q,
    uint8_t *__restrict__ sb, float *__restrict__ sg) {
  const int lane = threadIdx.x & 63;
  const int64_t row = row_begin + (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= row_end) return;  // whole wave exits together
  const int64_t nblk = C / 16;
  const uint16_t *xr = x + row * ld;
  uint32_t w[NB][8];
  uint32_t m = 0;
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    const int64_t blk = lane + 64 * b;
    if (blk < nblk) {
      const uint4 v0 = *reinterpret_cast<const uint4 *>(xr + blk * 16);
      const uint4 v1 = *reinterpret_cast<const uint4 *>(xr + blk * 16 + 8);
      w[b][0] = v0.x; w[b][1] = v0.y; w[b][2] = v0.z; w[b][3] = v0.w;
      w[b][4] = v1.x; w[b][5] = v1.y; w[b][6] = v1.z; w[b][7] = v1.w;
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) w[b][i] = 0;
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      m = max(m, w[b][i] & 0x7FFFu);
      m = max(m, (w[b][i] >> 16) & 0x7FFFu);
    }
  }
  float A;
  if (amax_ws) {
    A = __uint_as_float(amax_ws[row / rows_per_scale] << 16);
  } else {
    A = wave_max(__uint_as_float(m << 16));
  }
  const float s_g = __fdiv_rn(A, 2688.0f);  // one correctly rounded division
  if (lane == 0 && (amax_ws == nullptr || row % rows_per_scale == 0))
    sg[row / rows_per_scale] = s_g;
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    const int64_t blk = lane + 64 * b;
    if (blk < nblk) {
      uint2 packed;
      const uint32_t code = nvfp4_block(w[b], s_g, packed);
      *reinterpret_cast<uint2 *>(q + row * (C / 2) + blk * 8) = packed;
      sb[row * nblk + blk] = (uint8_t)code;
    }
  }
}

// Group maximum: each workgroup reduces a slab of rows of one group and
// folds it into amax_ws[group] (bf16 magnitude bits; integer order equals
// value order for non-negative finite values).
__global__ __launch_bounds__(256) void k_group_amax(
    const uint16_t *__restrict__ x, int64_t C, int64_t ld, int64_t row_begin,
    int64_t row_end, int64_t rows_per_scale, int64_t rows_per_wg,
    uint32_t *__restrict__ amax_ws) {
  const int64_t r0 = row_begin + (int64_t)blockIdx.x * rows_per_wg;
  int64_t r1 = r0 + rows_per_wg;
  if (r1 > row_end) r1 = row_end;
  const int64_t chunks = C / 8;
  uint32_t m = 0;
  for (int64_t r = r0; r < r1; ++r) {
    const uint16_t *xr = x + r * ld;
    for (int64_t c = threadIdx.x; c < chunks; c += 256) {
      const uint4 v = *reinterpret_cast<const uint4 *>(xr + c * 8);
      const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        m = max(m, w[i] & 0x7FFFu);
        m = max(m, (w[i] >> 16) & 0x7FFFu);
      }
    }
  }
  __shared__ uint32_t red[4];
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, o, 64));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
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

int64_t nvfp4_max_cols() { return 16 * 16 * 64; }

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
  // rows per amax workgroup: about 32 KB of input each, within one group
  int64_t rpw = (32768 / (C * 2));
  if (rpw < 1) rpw = 1;
  while (rows_per_scale % rpw) --rpw;
  for (int64_t g0 = 0; g0 < G; g0 += groups_per_chunk) {
    const int64_t g1 = (g0 + groups_per_chunk < G) ? g0 + groups_per_chunk : G;
    const int64_t rb = g0 * rows_per_scale, re = g1 * rows_per_scale;
    hipLaunchKernelGGL(k_group_amax, dim3((unsigned)((re - rb) / rpw)), dim3(256), 0, st, x, C,
                       ld, rb, re, rows_per_scale, rpw, ws);
    dispatch_rows(x, R, C, ld, rb, re, rows_per_scale, ws, q, sb, sg, st);
  }
  return hipGetLastError();
}

}  // namespace pqm
