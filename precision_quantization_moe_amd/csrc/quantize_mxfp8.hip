// quantize_mxfp8.hip -- MXFP8 row-wise and column-wise quantization in one
// HBM pass ("Towards Blackwell-Native 8-bit and 4-bit RL", Format
// background: MXFP8, and Recipe 1: training -- both copies are quantized
// independently from the high-precision input).
//
// One workgroup (256 lanes, 4 waves) owns a 128 x 128 tile of the bf16
// input.  Row-wise: each lane loads 16 bytes (8 elements); 4 neighbouring
// lanes hold one 1x32 block and reduce its maximum with two lane shuffles,
// then each lane writes its 8 E4M3 bytes.  The tile is staged in LDS and
// read down the columns for the 32x1 blocks; each lane then owns two
// columns of one 32-row block and writes 2 x 32 contiguous bytes of the
// transposed copy.
#include "pqm_device.hpp"
#include "pqm_internal.hpp"

namespace pqm {

constexpr int MX_TR = 128;  // tile rows
constexpr int MX_TC = 128;  // tile cols
constexpr int MX_PITCH = MX_TC * 2 + 16;  // LDS row pitch in bytes

template <bool ROW, bool COL>
__global__ __launch_bounds__(256) void k_quantize_mxfp8(
    const uint16_t *__restrict__ x, int64_t R, int64_t C, int64_t ld,
    uint8_t *__restrict__ q, uint8_t *__restrict__ s,
    uint8_t *__restrict__ qT, uint8_t *__restrict__ sT) {
  __shared__ __attribute__((aligned(16))) uint8_t tile[COL ? MX_TR * MX_PITCH : 16];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int64_t r0 = (int64_t)blockIdx.y * MX_TR;
  const int64_t c0 = (int64_t)blockIdx.x * MX_TC;

  // ---- phase 1: load, row-wise blocks, stage to LDS -------------------
  const int cchunk = lane & 15;  // 16 chunks of 8 elements per tile row
  const int64_t col = c0 + cchunk * 8;
  const bool col_ok = col < C;  // C % 32 == 0: whole blocks in or out
#pragma unroll 2
  for (int it = 0; it < MX_TR / 16; ++it) {
    const int rl = it * 16 + wave * 4 + (lane >> 4);
    const int64_t row = r0 + rl;
    uint4 v = make_uint4(0, 0, 0, 0);
    const bool ok = col_ok && row < R;
    if (ok) v = *reinterpret_cast<const uint4 *>(x + row * ld + col);
    if (COL) *reinterpret_cast<uint4 *>(tile + rl * MX_PITCH + cchunk * 16) = v;
    if (ROW) {
      // block maximum over 4 lanes (bf16 magnitude bits compare as integers)
      uint32_t m = 0;
      const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        m = max(m, w[i] & 0x7FFFu);
        m = max(m, (w[i] >> 16) & 0x7FFFu);
      }
      m = max(m, (uint32_t)__shfl_xor((int)m, 1, 64));
      m = max(m, (uint32_t)__shfl_xor((int)m, 2, 64));
      const uint32_t sb = mx_scale_byte(m);
      const float inv = mx_inv_scale(sb);
      uint32_t out[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        uint32_t b0 = mx_encode(w[2 * h] & 0xFFFFu, inv);
        uint32_t b1 = mx_encode(w[2 * h] >> 16, inv);
        uint32_t b2 = mx_encode(w[2 * h + 1] & 0xFFFFu, inv);
        uint32_t b3 = mx_encode(w[2 * h + 1] >> 16, inv);
        out[h] = b0 | (b1 << 8) | (b2 << 16) | (b3 << 24);
      }
      if (ok) {
        *reinterpret_cast<uint2 *>(q + row * C + col) = make_uint2(out[0], out[1]);
        if ((lane & 3) == 0) s[row * (C / 32) + col / 32] = (uint8_t)sb;
      }
    }
  }
  if (!COL) return;
  __syncthreads();

  // ---- phase 2: column-wise 32x1 blocks from LDS ----------------------
  const int cp = tid & 63;   // column pair within the tile
  const int rb = tid >> 6;   // 32-row block within the tile
  const int64_t cg = c0 + 2 * cp;
  const int64_t rg = r0 + rb * 32;
  if (cg >= C || rg >= R) return;  // R % 32 == 0, C % 32 == 0
  uint32_t w[32];
#pragma unroll
  for (int i = 0; i < 32; ++i)
    w[i] = *reinterpret_cast<const uint32_t *>(tile + (rb * 32 + i) * MX_PITCH + cp * 4);
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    uint32_t m = 0;
#pragma unroll
    for (int i = 0; i < 32; ++i) m = max(m, (w[i] >> (16 * h)) & 0x7FFFu);
    const uint32_t sb = mx_scale_byte(m);
    const float inv = mx_inv_scale(sb);
    uint32_t o[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      uint32_t acc = 0;
#pragma unroll
      for (int k = 0; k < 4; ++k)
        acc |= mx_encode((w[4 * j + k] >> (16 * h)) & 0xFFFFu, inv) << (8 * k);
      o[j] = acc;
    }
    uint8_t *dst = qT + (cg + h) * R + rg;
    reinterpret_cast<uint4 *>(dst)[0] = make_uint4(o[0], o[1], o[2], o[3]);
    reinterpret_cast<uint4 *>(dst)[1] = make_uint4(o[4], o[5], o[6], o[7]);
    sT[(cg + h) * (R / 32) + rg / 32] = (uint8_t)sb;
  }
}

hipError_t launch_quantize_mxfp8(const uint16_t *x, int64_t R, int64_t C, int64_t ld,
                                 uint8_t *q, uint8_t *s, uint8_t *qT, uint8_t *sT,
                                 hipStream_t st) {
  if (R == 0 || C == 0) return hipSuccess;
  dim3 grid((unsigned)((C + MX_TC - 1) / MX_TC), (unsigned)((R + MX_TR - 1) / MX_TR));
  const bool row = q != nullptr, col = qT != nullptr;
  if (row && col)
    hipLaunchKernelGGL((k_quantize_mxfp8<true, true>), grid, dim3(256), 0, st, x, R, C, ld, q, s, qT, sT);
  else if (row)
    hipLaunchKernelGGL((k_quantize_mxfp8<true, false>), grid, dim3(256), 0, st, x, R, C, ld, q, s, qT, sT);
  else
    hipLaunchKernelGGL((k_quantize_mxfp8<false, true>), grid, dim3(256), 0, st, x, R, C, ld, q, s, qT, sT);
  return hipGetLastError();
}

}  // namespace pqm
