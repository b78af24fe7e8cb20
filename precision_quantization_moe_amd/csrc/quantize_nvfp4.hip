// quantize_nvfp4.hip -- NVFP4 quantization with an online FP32 outer scale
// ("Towards Blackwell-Native 8-bit and 4-bit RL", Format background: NVFP4
// and Recipe 2: per-token activation scaling; "miniTE technical report",
// 2.2 decode x^ = q * s_b * s_g and 5.6 gs = gamax / 2688).
//
// Per-token scope: one wave owns one row.  The row is read once into
// registers with 16-byte loads (one 1x16 block per lane per step), its
// maximum is reduced across the wave, and all three outputs (packed E2M1,
// E4M3 block scales, FP32 token scale) are written from registers.  Both
// roundings run on binary32 brackets whose rare disagreements are settled by
// the sign of A - 2688 s_g (see nvfp4_block); no per-element division.
//
// Group scope (one outer scale for rows_per_scale rows, e.g. an expert's
// fused gate/up weight): the group maximum is reduced with atomicMax on the
// bf16 magnitude bits into AMAX_SLOTS words of the group, each in its own
// 128-byte line (same-line atomics from hundreds of workgroups serialise
// and cost as much as the whole read); the quantizing waves fold the slots.
// Groups go in chunks of about 64 MB, and one launch both quantizes chunk
// j-1 and reduces the maxima of chunk j, so chunk j-1's second read is
// served from the Infinity Cache while chunk j streams in from HBM.
#include "nvfp4_encode.hpp"
#include "pqm_device.hpp"
#include "pqm_internal.hpp"

namespace pqm {

// Group-maximum slots per group and their spacing in 32-bit words.
constexpr int AMAX_SLOTS = 16;
constexpr int AMAX_STRIDE = 32;

// One wave per row: lane l owns the 1x16 blocks l + 64 j (two 16-byte loads
// each), all issued before any use; NB blocks per lane (cols <= 1024 NB).
// When amax_ws is non-null the outer scale comes from the group's slot
// words (row / rows_per_scale) instead of the row.
template <int NB>
__device__ __forceinline__ void nvfp4_row_wave(const uint16_t *__restrict__ x, uint32_t C,
                                               int64_t ld, uint32_t row, uint32_t rows_per_scale,
                                               const uint32_t *__restrict__ amax_ws,
                                               uint8_t *__restrict__ q, uint8_t *__restrict__ sb,
                                               float *__restrict__ sg) {
  const int lane = threadIdx.x & 63;
  const uint32_t nblk = C / 16;
  const uint16_t *xr = x + (int64_t)row * ld;
  uint32_t w[NB][8];
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    const uint32_t blk = lane + 64 * b;
    uint4 v0 = make_uint4(0, 0, 0, 0), v1 = v0;
    if (blk < nblk) {
      v0 = *reinterpret_cast<const uint4 *>(xr + blk * 16);
      v1 = *reinterpret_cast<const uint4 *>(xr + blk * 16 + 8);
    }
    w[b][0] = v0.x; w[b][1] = v0.y; w[b][2] = v0.z; w[b][3] = v0.w;
    w[b][4] = v1.x; w[b][5] = v1.y; w[b][6] = v1.z; w[b][7] = v1.w;
  }
  const uint32_t grp = amax_ws ? row / rows_per_scale : row;
  float A;
  if (amax_ws) {
    uint32_t m = lane < AMAX_SLOTS ? amax_ws[((size_t)grp * AMAX_SLOTS + lane) * AMAX_STRIDE] : 0u;
#pragma unroll
    for (int o = AMAX_SLOTS / 2; o >= 1; o >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, o, 64));
    A = __uint_as_float((uint32_t)__builtin_amdgcn_readfirstlane((int)m) << 16);
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
  const Nvfp4Row rc = nvfp4_row(A);
  if (lane == 0 && (amax_ws == nullptr || row == grp * rows_per_scale)) sg[grp] = rc.s_g;
  uint8_t *qr = q + (int64_t)row * (C / 2);
  uint8_t *sbr = sb + (int64_t)row * nblk;
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    if (64u * b < nblk) {  // uniform: the exact path's ballot needs the wave
      const uint32_t blk = lane + 64 * b;
      uint32_t code;
      const uint2 packed = nvfp4_block(w[b], rc, &code);
      if (blk < nblk) {
        typedef uint32_t u2v __attribute__((ext_vector_type(2)));
        __builtin_nontemporal_store(u2v{packed.x, packed.y}, reinterpret_cast<u2v *>(qr + blk * 8));
        sbr[blk] = (uint8_t)code;
      }
    }
  }
}

// D = bf16(silu(gate) up p) (pqm_swiglu_prob) fused with the per-token
// NVFP4 encoding of D, the FC2 operand ("miniTE technical report", 5.3-5.4:
// the activation times the router probability is quantized where it is
// produced, and its per-token amax needs no separate pass).  One wave per
// row of D: lane l owns the 1x16 D blocks l + 64 b, whose gate and up values
// are the 16 columns 16 (l + 64 b) .. of C's two halves; the row maximum,
// s_g and the blocks are then exactly those of the per-token quantizer.
// The loads are unconditional (blocks past the row re-read its last block
// and are then zeroed), so that no load waits at a branch join.
template <int NB>
__global__ __launch_bounds__(256) void k_swiglu_quant_nvfp4(
    const uint16_t *__restrict__ c, const float *__restrict__ prob,
    const int32_t *__restrict__ src, uint32_t rows, uint32_t I, uint16_t *__restrict__ d,
    uint8_t *__restrict__ q, uint8_t *__restrict__ sb, float *__restrict__ sg) {
  const uint32_t row = blockIdx.x * 4u + (threadIdx.x >> 6);
  if (row >= rows) return;  // whole wave exits together
  const int lane = threadIdx.x & 63;
  const uint32_t nblk = I / 16;
  const float p = prob[src ? src[row] : (int32_t)row];
  const uint16_t *cr = c + (int64_t)row * 2 * I;
  uint4 gv[NB][2], uv[NB][2];
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    const uint32_t blk = min(lane + 64u * b, nblk - 1u);
    gv[b][0] = *reinterpret_cast<const uint4 *>(cr + blk * 16);
    gv[b][1] = *reinterpret_cast<const uint4 *>(cr + blk * 16 + 8);
    uv[b][0] = *reinterpret_cast<const uint4 *>(cr + I + blk * 16);
    uv[b][1] = *reinterpret_cast<const uint4 *>(cr + I + blk * 16 + 8);
  }
  uint32_t w[NB][8];
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    const bool ok = lane + 64u * b < nblk;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const uint32_t gw[4] = {gv[b][h].x, gv[b][h].y, gv[b][h].z, gv[b][h].w};
      const uint32_t uw[4] = {uv[b][h].x, uv[b][h].y, uv[b][h].z, uv[b][h].w};
#pragma unroll
      for (int k = 0; k < 4; ++k)
        w[b][4 * h + k] = ok ? pk_bf16_rne(swiglu_f32(bf16_lo_f32(gw[k]), bf16_lo_f32(uw[k]), p),
                                           swiglu_f32(bf16_hi_f32(gw[k]), bf16_hi_f32(uw[k]), p))
                             : 0u;
    }
  }
  uint32_t m = 0;
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int i = 0; i < 8; ++i) m = pk_max_u16(m, w[b][i] & 0x7FFF7FFFu);
  m = max(m & 0xFFFFu, m >> 16);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, o, 64));
  const Nvfp4Row rc = nvfp4_row(__uint_as_float(m << 16));
  if (lane == 0) sg[row] = rc.s_g;
  uint8_t *qr = q + (int64_t)row * (I / 2);
  uint8_t *sbr = sb + (int64_t)row * nblk;
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    if (64u * b < nblk) {  // uniform: the exact path's ballot needs the wave
      const uint32_t blk = lane + 64u * b;
      uint32_t code;
      const uint2 packed = nvfp4_block(w[b], rc, &code);
      if (blk < nblk) {
        typedef uint32_t u2v __attribute__((ext_vector_type(2)));
        __builtin_nontemporal_store(u2v{packed.x, packed.y}, reinterpret_cast<u2v *>(qr + blk * 8));
        sbr[blk] = (uint8_t)code;
        if (d) {
          uint16_t *dr = d + (int64_t)row * I + blk * 16;
          *reinterpret_cast<uint4 *>(dr) = make_uint4(w[b][0], w[b][1], w[b][2], w[b][3]);
          *reinterpret_cast<uint4 *>(dr + 8) = make_uint4(w[b][4], w[b][5], w[b][6], w[b][7]);
        }
      }
    }
  }
}

hipError_t launch_swiglu_quant_nvfp4(const uint16_t *c, const float *prob, const int32_t *src,
                                     int64_t M, int64_t I, uint16_t *d, uint8_t *q, uint8_t *sb,
                                     float *sg, hipStream_t st) {
  if (M == 0 || I == 0) return hipSuccess;
  const dim3 grid((unsigned)((M + 3) / 4));
  const int64_t per_lane = (I / 16 + 63) / 64;
#define PQM_SQ(NB)                                                                        \
  hipLaunchKernelGGL((k_swiglu_quant_nvfp4<NB>), grid, dim3(256), 0, st, c, prob, src,  \
                     (uint32_t)M, (uint32_t)I, d, q, sb, sg)
  if (per_lane <= 1) PQM_SQ(1);
  else if (per_lane <= 2) PQM_SQ(2);
  else if (per_lane <= 4) PQM_SQ(4);
  else if (per_lane <= 8) PQM_SQ(8);
  else PQM_SQ(16);
#undef PQM_SQ
  return hipGetLastError();
}

// Per-token scope: workgroup b quantizes rows 4b .. 4b+3, one per wave.
template <int NB>
__global__ __launch_bounds__(256) void k_quantize_nvfp4_rows(
    const uint16_t *__restrict__ x, uint32_t C, int64_t ld, uint32_t rows,
    uint8_t *__restrict__ q, uint8_t *__restrict__ sb, float *__restrict__ sg) {
  const uint32_t row = blockIdx.x * 4u + (threadIdx.x >> 6);
  if (row >= rows) return;  // whole wave exits together
  nvfp4_row_wave<NB>(x, C, ld, row, 1u, nullptr, q, sb, sg);
}

// Group maximum of rows [r0, r1) (all in one group; wave w takes rows w,
// w+4, ...; 16-byte loads, packed 16-bit max), folded with one atomicMax
// into slot `slot` of the group (bf16 magnitude bits: integer order equals
// value order for non-negative finite values).  Whole workgroup.
template <int NB>
__device__ __forceinline__ void group_amax_wg(const uint16_t *__restrict__ x, int64_t C,
                                              int64_t ld, int64_t r0, int64_t r1,
                                              int64_t rows_per_scale, int slot,
                                              uint32_t *__restrict__ amax_ws) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t nblk = C / 16;
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
    atomicMax(&amax_ws[((r0 / rows_per_scale) * AMAX_SLOTS + slot) * AMAX_STRIDE], m);
  }
}

// One step of the group-scope pipeline: quantize rows [qb, qe) (whose group
// maxima are complete) and reduce the group maxima of rows [ab, ae), in one
// launch.  Workgroups alternate between the two roles while both have work,
// so the reduction's HBM reads overlap the quantization's cache-served
// re-reads.  nq / na: workgroups of each role (4 rows, resp. rpw rows each).
struct Nvfp4Step {
  int64_t qb, qe, ab, ae, rpw;
  uint32_t nq, na;
};

template <int NB>
__global__ __launch_bounds__(256) void k_nvfp4_group_step(
    const uint16_t *__restrict__ x, uint32_t C, int64_t ld, uint32_t rows_per_scale,
    Nvfp4Step p, uint32_t *__restrict__ amax_ws, uint8_t *__restrict__ q,
    uint8_t *__restrict__ sb, float *__restrict__ sg) {
  const uint32_t b = blockIdx.x, both = min(p.nq, p.na);
  bool quant;
  uint32_t idx;
  if (b < 2u * both) {
    quant = (b & 1u) == 0u;
    idx = b >> 1;
  } else {
    quant = p.nq > p.na;
    idx = b - both;
  }
  if (quant) {
    const int64_t row = p.qb + (int64_t)idx * 4 + (threadIdx.x >> 6);
    if (row >= p.qe) return;  // whole wave exits together
    nvfp4_row_wave<NB>(x, C, ld, (uint32_t)row, rows_per_scale, amax_ws, q, sb, sg);
  } else {
    const int64_t r0 = p.ab + (int64_t)idx * p.rpw;
    const int64_t r1 = r0 + p.rpw < p.ae ? r0 + p.rpw : p.ae;
    group_amax_wg<NB>(x, C, ld, r0, r1, rows_per_scale, (int)(idx % AMAX_SLOTS), amax_ws);
  }
}

__global__ void k_fill_u32(uint32_t *p, int64_t n, uint32_t v) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

template <int NB>
static void launch_nb(const uint16_t *x, int64_t R, int64_t C, int64_t ld, int64_t rps,
                      const Nvfp4Step *step, uint32_t *ws, uint8_t *q, uint8_t *sb, float *sg,
                      hipStream_t st) {
  if (!step) {
    const unsigned grid = (unsigned)((R + 3) / 4);
    hipLaunchKernelGGL((k_quantize_nvfp4_rows<NB>), dim3(grid), dim3(256), 0, st, x,
                       (uint32_t)C, ld, (uint32_t)R, q, sb, sg);
  } else {
    const unsigned grid = step->nq + step->na;
    hipLaunchKernelGGL((k_nvfp4_group_step<NB>), dim3(grid), dim3(256), 0, st, x, (uint32_t)C,
                       ld, (uint32_t)rps, *step, ws, q, sb, sg);
  }
}

// step == nullptr: the per-token kernel over all R rows.
static void dispatch_nb(const uint16_t *x, int64_t R, int64_t C, int64_t ld, int64_t rps,
                        const Nvfp4Step *step, uint32_t *ws, uint8_t *q, uint8_t *sb,
                        float *sg, hipStream_t st) {
  const int64_t per_lane = (C / 16 + 63) / 64;
  if (per_lane <= 1) launch_nb<1>(x, R, C, ld, rps, step, ws, q, sb, sg, st);
  else if (per_lane <= 2) launch_nb<2>(x, R, C, ld, rps, step, ws, q, sb, sg, st);
  else if (per_lane <= 4) launch_nb<4>(x, R, C, ld, rps, step, ws, q, sb, sg, st);
  else if (per_lane <= 8) launch_nb<8>(x, R, C, ld, rps, step, ws, q, sb, sg, st);
  else launch_nb<16>(x, R, C, ld, rps, step, ws, q, sb, sg, st);
}

int64_t nvfp4_max_cols() { return 16 * 1024; }

size_t nvfp4_workspace_bytes(int64_t R, int64_t rows_per_scale) {
  if (rows_per_scale <= 1 || R == 0) return 0;
  return (size_t)(R / rows_per_scale) * AMAX_SLOTS * AMAX_STRIDE * sizeof(uint32_t);
}

// Group scope in chunks of whole groups of about chunk_bytes of input:
// launch j quantizes chunk j-1 and reduces the maxima of chunk j.
hipError_t launch_quantize_nvfp4_chunked(const uint16_t *x, int64_t R, int64_t C, int64_t ld,
                                         int64_t rows_per_scale, uint8_t *q, uint8_t *sb,
                                         float *sg, void *workspace, int64_t chunk_bytes,
                                         hipStream_t st) {
  uint32_t *ws = static_cast<uint32_t *>(workspace);
  const int64_t G = R / rows_per_scale;
  const int64_t nws = G * AMAX_SLOTS * AMAX_STRIDE;
  hipLaunchKernelGGL(k_fill_u32, dim3((unsigned)((nws + 255) / 256)), dim3(256), 0, st, ws, nws,
                     0u);
  const int64_t group_bytes = rows_per_scale * C * 2;
  int64_t gpc = chunk_bytes / (group_bytes > 0 ? group_bytes : 1);  // groups per chunk
  if (gpc < 1) gpc = 1;
  // rows per reducing workgroup: about 16 KB of input (at least one row per
  // wave), dividing rows_per_scale so that a workgroup stays in one group
  int64_t rpw = 16384 / (C * 2);
  if (rpw < 4) rpw = 4;
  while (rows_per_scale % rpw) --rpw;
  const int64_t rows_per_chunk = gpc * rows_per_scale;
  const int64_t nchunk = (G + gpc - 1) / gpc;
  for (int64_t j = 0; j <= nchunk; ++j) {
    Nvfp4Step p{0, 0, 0, 0, rpw, 0u, 0u};
    if (j > 0) {
      p.qb = (j - 1) * rows_per_chunk;
      p.qe = p.qb + rows_per_chunk < R ? p.qb + rows_per_chunk : R;
      p.nq = (uint32_t)((p.qe - p.qb + 3) / 4);
    }
    if (j < nchunk) {
      p.ab = j * rows_per_chunk;
      p.ae = p.ab + rows_per_chunk < R ? p.ab + rows_per_chunk : R;
      p.na = (uint32_t)((p.ae - p.ab) / rpw);
    }
    dispatch_nb(x, R, C, ld, rows_per_scale, &p, ws, q, sb, sg, st);
  }
  return hipGetLastError();
}

hipError_t launch_quantize_nvfp4(const uint16_t *x, int64_t R, int64_t C, int64_t ld,
                                 int64_t rows_per_scale, uint8_t *q, uint8_t *sb, float *sg,
                                 void *workspace, hipStream_t st) {
  if (R == 0 || C == 0) return hipSuccess;
  if (rows_per_scale == 1) {
    dispatch_nb(x, R, C, ld, 1, nullptr, nullptr, q, sb, sg, st);
    return hipGetLastError();
  }
  return launch_quantize_nvfp4_chunked(x, R, C, ld, rows_per_scale, q, sb, sg, workspace,
                                       (int64_t)64 << 20, st);
}

}  // namespace pqm
