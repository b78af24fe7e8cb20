// quantize_mxfp8.hip -- MXFP8 row-wise and column-wise quantization in one
// HBM pass ("Towards Blackwell-Native 8-bit and 4-bit RL", Format
// background: MXFP8, and Recipe 1: training -- both copies are quantized
// independently from the high-precision input).
//
// One workgroup (256 lanes) per 128 x 128 tile of the bf16 input (the
// hardware dispatcher balances tiles over the CUs; a persistent loop left a
// partial last round); all of the tile's 16-byte loads are issued first.
//  1. Row-wise: 4 neighbouring lanes hold one 1x32 block (16-byte loads),
//     reduce its maximum (packed 16-bit max, two lane shuffles), take the
//     scale exponent from the maximum's bf16 bits and convert the elements
//     two per instruction (scaled bf16 -> E4M3 conversion).  The bf16 tile
//     goes to LDS.
//  2. Column-wise: each lane reads two columns of one 32-row block from
//     LDS, pairs consecutive rows with a byte permute and encodes them.
//  3. Both encoded copies (16 KB each) and their scale bytes are staged in
//     LDS, then written with 16-byte stores in which 8 consecutive lanes
//     cover one 128-byte line of q (a tile row) or of the transposed copy
//     (a tile column); the 4 scale bytes of a row / column go out as one
//     32-bit store.  Writing the transposed copy directly from the encoding
//     lanes (32 bytes per lane, each to a different line) was the dominant
//     cost before this staging.
#include "pqm_device.hpp"
#include "pqm_internal.hpp"

namespace pqm {

constexpr int MX_T = 128;                 // tile rows = tile cols
constexpr int MX_PITCH = MX_T * 2 + 16;   // LDS row pitch of the bf16 tile
constexpr int MX_IT = MX_T / 16;          // 16-byte loads per lane per tile
constexpr int MX_OP = MX_T + 16;          // LDS pitch of a staged byte row
// staging layout inside the (reused) bf16 tile buffer, in bytes
constexpr int MX_OQ = 0;                         // q   [128 rows][MX_OP]
constexpr int MX_OQT = MX_T * MX_OP;             // qT  [128 cols][MX_OP]
constexpr int MX_OS = 2 * MX_T * MX_OP;          // s   [128 rows][4]
constexpr int MX_OST = MX_OS + MX_T * 4;         // sT  [128 cols][4]
constexpr int MX_STAGE = MX_OST + MX_T * 4;
constexpr int MX_LDS = MX_T * MX_PITCH > MX_STAGE ? MX_T * MX_PITCH : MX_STAGE;

struct MxTile {
  uint4 v[MX_IT];
};

__device__ __forceinline__ void mx_load_tile(const uint16_t *__restrict__ x, int64_t R,
                                             int64_t C, int64_t ld, int64_t ntc, int64_t t,
                                             MxTile &tl) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t r0 = (t / ntc) * MX_T, c0 = (t % ntc) * MX_T;
  const int64_t col = c0 + (lane & 15) * 8;
#pragma unroll
  for (int it = 0; it < MX_IT; ++it) {
    const int64_t row = r0 + it * 16 + wave * 4 + (lane >> 4);
    tl.v[it] = make_uint4(0, 0, 0, 0);
    if (col < C && row < R) tl.v[it] = *reinterpret_cast<const uint4 *>(x + row * ld + col);
  }
}

template <bool ROW, bool COL>
__global__ __launch_bounds__(256) void k_quantize_mxfp8(
    const uint16_t *__restrict__ x, int64_t R, int64_t C, int64_t ld, int64_t ntc,
    int64_t ntiles, uint8_t *__restrict__ q, uint8_t *__restrict__ s,
    uint8_t *__restrict__ qT, uint8_t *__restrict__ sT) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[MX_LDS];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int cchunk = lane & 15;  // 16 chunks of 8 elements per tile row
  const bool s_vec = (C % 128) == 0;   // row scales of a tile: one aligned word
  const bool sT_vec = (R % 128) == 0;  // column scales of a tile: one aligned word

  const int64_t t = blockIdx.x;
  {
    MxTile cur;
    mx_load_tile(x, R, C, ld, ntc, t, cur);
    const int64_t r0 = (t / ntc) * MX_T, c0 = (t % ntc) * MX_T;

    // ---- 1. row-wise encode from registers; bf16 tile to LDS ------------
    uint2 rq[MX_IT];
    uint32_t rs[MX_IT];
#pragma unroll
    for (int it = 0; it < MX_IT; ++it) {
      const int rl = it * 16 + wave * 4 + (lane >> 4);
      const uint4 v = cur.v[it];
      if (COL) *reinterpret_cast<uint4 *>(lds + rl * MX_PITCH + cchunk * 16) = v;
      if (ROW) {
        uint32_t m = pk_max_u16(pk_max_u16(v.x & 0x7FFF7FFFu, v.y & 0x7FFF7FFFu),
                                pk_max_u16(v.z & 0x7FFF7FFFu, v.w & 0x7FFF7FFFu));
        m = max(m & 0xFFFFu, m >> 16);
        m = max(m, (uint32_t)__shfl_xor((int)m, 1, 64));
        m = max(m, (uint32_t)__shfl_xor((int)m, 2, 64));
        const uint32_t sb = mx_scale_byte(m);
        rq[it] = make_uint2(mx_encode4(v.x, v.y, sb), mx_encode4(v.z, v.w, sb));
        rs[it] = sb;
      }
    }
    // ---- 2. column-wise encode from LDS ---------------------------------
    uint32_t co[2][8];
    uint32_t csb[2] = {0, 0};
    const int cp = tid & 63;  // column pair
    const int rb = tid >> 6;  // 32-row block
    if (COL) {
      __syncthreads();
      uint32_t w[32];
#pragma unroll
      for (int i = 0; i < 32; ++i)
        w[i] = *reinterpret_cast<const uint32_t *>(lds + (rb * 32 + i) * MX_PITCH + cp * 4);
      uint32_t m = 0;
#pragma unroll
      for (int i = 0; i < 32; ++i) m = pk_max_u16(m, w[i] & 0x7FFF7FFFu);
      csb[0] = mx_scale_byte(m & 0xFFFFu);
      csb[1] = mx_scale_byte(m >> 16);
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const uint32_t sel = h ? 0x07060302u : 0x05040100u;  // column h, rows i, i+1
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const uint32_t p0 = __builtin_amdgcn_perm(w[4 * j + 1], w[4 * j], sel);
          const uint32_t p1 = __builtin_amdgcn_perm(w[4 * j + 3], w[4 * j + 2], sel);
          co[h][j] = mx_encode4(p0, p1, csb[h]);
        }
      }
    }
    __syncthreads();  // the bf16 tile is no longer read: reuse it for staging
    // ---- 3. stage both copies and scales --------------------------------
    if (ROW) {
#pragma unroll
      for (int it = 0; it < MX_IT; ++it) {
        const int rl = it * 16 + wave * 4 + (lane >> 4);
        *reinterpret_cast<uint2 *>(lds + MX_OQ + rl * MX_OP + cchunk * 8) = rq[it];
        if ((lane & 3) == 0) lds[MX_OS + rl * 4 + (cchunk >> 2)] = (uint8_t)rs[it];
      }
    }
    if (COL) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        uint8_t *dst = lds + MX_OQT + (2 * cp + h) * MX_OP + rb * 32;
        reinterpret_cast<uint4 *>(dst)[0] = make_uint4(co[h][0], co[h][1], co[h][2], co[h][3]);
        reinterpret_cast<uint4 *>(dst)[1] = make_uint4(co[h][4], co[h][5], co[h][6], co[h][7]);
        lds[MX_OST + (2 * cp + h) * 4 + rb] = (uint8_t)csb[h];
      }
    }
    __syncthreads();
    // ---- 4. coalesced stores ---------------------------------------------
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int c = tid + 256 * k;       // 16-byte chunk: 8 per staged row
      const int r = c >> 3, b = (c & 7) * 16;
      if (ROW) {
        const int64_t row = r0 + r, col = c0 + b;
        if (row < R && col < C)
          *reinterpret_cast<uint4 *>(q + row * C + col) =
              *reinterpret_cast<const uint4 *>(lds + MX_OQ + r * MX_OP + b);
      }
      if (COL) {
        const int64_t colg = c0 + r, rowg = r0 + b;
        if (colg < C && rowg < R)
          *reinterpret_cast<uint4 *>(qT + colg * R + rowg) =
              *reinterpret_cast<const uint4 *>(lds + MX_OQT + r * MX_OP + b);
      }
    }
    if (tid < MX_T) {
      const int r = tid;
      if (ROW && r0 + r < R) {
        const uint32_t w4 = *reinterpret_cast<const uint32_t *>(lds + MX_OS + r * 4);
        uint8_t *dst = s + (r0 + r) * (C / 32) + c0 / 32;
        if (s_vec) {
          *reinterpret_cast<uint32_t *>(dst) = w4;
        } else {
          for (int j = 0; j < 4 && c0 + 32 * j < C; ++j) dst[j] = (uint8_t)(w4 >> (8 * j));
        }
      }
      if (COL && c0 + r < C) {
        const uint32_t w4 = *reinterpret_cast<const uint32_t *>(lds + MX_OST + r * 4);
        uint8_t *dst = sT + (c0 + r) * (R / 32) + r0 / 32;
        if (sT_vec) {
          *reinterpret_cast<uint32_t *>(dst) = w4;
        } else {
          for (int j = 0; j < 4 && r0 + 32 * j < R; ++j) dst[j] = (uint8_t)(w4 >> (8 * j));
        }
      }
    }
  }
}

hipError_t launch_quantize_mxfp8(const uint16_t *x, int64_t R, int64_t C, int64_t ld,
                                 uint8_t *q, uint8_t *s, uint8_t *qT, uint8_t *sT,
                                 hipStream_t st) {
  if (R == 0 || C == 0) return hipSuccess;
  const int64_t ntc = (C + MX_T - 1) / MX_T, ntr = (R + MX_T - 1) / MX_T;
  const int64_t ntiles = ntc * ntr;
  const bool row = q != nullptr, col = qT != nullptr;
  const void *kern = row && col ? (const void *)k_quantize_mxfp8<true, true>
                     : row      ? (const void *)k_quantize_mxfp8<true, false>
                                : (const void *)k_quantize_mxfp8<false, true>;
  (void)kern;
  const dim3 grid((unsigned)ntiles);
  if (row && col)
    hipLaunchKernelGGL((k_quantize_mxfp8<true, true>), grid, dim3(256), 0, st, x, R, C, ld, ntc,
                       ntiles, q, s, qT, sT);
  else if (row)
    hipLaunchKernelGGL((k_quantize_mxfp8<true, false>), grid, dim3(256), 0, st, x, R, C, ld,
                       ntc, ntiles, q, s, qT, sT);
  else
    hipLaunchKernelGGL((k_quantize_mxfp8<false, true>), grid, dim3(256), 0, st, x, R, C, ld,
                       ntc, ntiles, q, s, qT, sT);
  return hipGetLastError();
}

}  // namespace pqm
