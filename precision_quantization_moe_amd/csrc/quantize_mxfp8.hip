// quantize_mxfp8.hip -- MXFP8 row-wise and column-wise quantization in one
// HBM pass ("Towards Blackwell-Native 8-bit and 4-bit RL", Format
// background: MXFP8, and Recipe 1: training -- both copies are quantized
// independently from the high-precision input).
//
// The input is cut into 128 x 128 tiles.  Within a tile, wave w owns the rows
// 32w .. 32w+31, which is exactly one 32-row column block; lane
// (r = lane / 16, c = lane % 16) loads the 8 columns 8c .. 8c+7 of the 8
// consecutive rows 32w + 8r + i (i = 0..7) with 16-byte loads (each load
// instruction covers 4 whole 256-byte row segments).  Both block kinds are
// then reduced without LDS:
//  * row block (1 x 32): the 4 lanes c = 4j .. 4j+3 of one row -- packed
//    16-bit maxima of the magnitude bits, then two quad permutes (DPP);
//  * column block (32 x 1): the lane's 8 rows in registers, then the 4 lanes
//    r = 0..3 (lane swaps across 16 and 32 lanes).
// The scale byte comes from the block maximum's bf16 bits and the elements
// are converted two per instruction by the scaled bf16 -> E4M3 conversion,
// which takes the E8M0 byte as its scale exponent (byte 0 included): row
// pairs are neighbouring columns, column pairs neighbouring rows (one byte
// permute).  The lane's row-wise bytes (8 per row) are stored straight to q
// (16 lanes per 128-byte line); its column-wise bytes (8 consecutive rows of
// each of its 8 columns) are staged in LDS and leave as whole lines of the
// transposed copy.  Scale bytes are gathered in LDS and leave as one 32-bit
// word per row (4 row blocks) and per column and tile (4 column blocks).
//
// Interior workgroups take MX_VT vertically adjacent tiles (all loads issued
// first, the transposed copy leaving in runs of MX_VT * 128 bytes); tiles cut
// by the input's edge (rows or columns not a multiple of 128, or a band left
// over from the grouping) run in a second, bounds-checked launch of single
// tiles.  With one tile per workgroup (52-59 registers, 17 KB of LDS) all
// 2048 tiles of a 16384 x 2048 input are resident at once.  Workgroups take tiles in row-major
// order, so consecutively dispatched workgroups read neighbouring segments of
// the same rows (dealing contiguous tile ranges to each XCD instead measured
// slower on MI355X).
#include "pqm_device.hpp"
#include "pqm_internal.hpp"

namespace pqm {

constexpr int MX_T = 128;  // tile rows = tile cols

// The E8M0 scale of a block as the binary32 bits (b << 23) of 2^(b-127),
// from the bf16 magnitude bits of the block maximum held in the low (lo) or
// high (hi) 16 bits of m: b = max(0, ((amax + 0x1F) >> 7) - 8) as in
// mx_scale_byte, computed in place in the exponent field with a saturating
// subtraction.
__device__ __forceinline__ uint32_t mx_scale_bits_lo(uint32_t m) {
  return __builtin_elementwise_sub_sat(((m + 0x1Fu) << 16) & 0x7F800000u, 0x04000000u);
}
__device__ __forceinline__ uint32_t mx_scale_bits_hi(uint32_t m) {
  return __builtin_elementwise_sub_sat((m + 0x1F0000u) & 0x7F800000u, 0x04000000u);
}

// cvt4_e4m3_bf16 writing into the register of `old`, a value that is dead
// afterwards (all four bytes are overwritten), so that no zeroed register
// has to be set up for the partial writes of the conversions.
__device__ __forceinline__ uint32_t cvt4_e4m3_bf16_into(uint32_t old, uint32_t w0, uint32_t w1,
                                                        uint32_t scale_bits) {
  const float scale = __uint_as_float(scale_bits);
  pqm_v2s r = __builtin_bit_cast(pqm_v2s, old);
  r = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(r, __builtin_bit_cast(pqm_v2bf, w0), scale,
                                                 false);
  r = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(r, __builtin_bit_cast(pqm_v2bf, w1), scale,
                                                 true);
  return __builtin_bit_cast(uint32_t, r);
}

// Maximum over the lane pair {l, l ^ 1}, {l, l ^ 2} (quad permutes).
__device__ __forceinline__ uint32_t max_xor1(uint32_t m) {
  return max(m, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)m, 0xB1, 0xF, 0xF, false));
}
__device__ __forceinline__ uint32_t max_xor2(uint32_t m) {
  return max(m, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)m, 0x4E, 0xF, 0xF, false));
}
// Packed 16-bit maximum over the lanes l and l ^ 16, then l ^ 32.  The
// gfx950 lane swaps exchange the odd 16-lane rows of the first operand with
// the even rows of the second (permlane16) and the upper half of the first
// with the lower half of the second (permlane32); with both operands m, the
// maximum of the two results is max(m[l], m[l ^ 16]) (resp. l ^ 32) in every
// lane.
__device__ __forceinline__ uint32_t pk_max_xor16(uint32_t m) {
  const auto p = __builtin_amdgcn_permlane16_swap(m, m, false, false);
  return pk_max_u16(p[0], p[1]);
}
__device__ __forceinline__ uint32_t pk_max_xor32(uint32_t m) {
  const auto p = __builtin_amdgcn_permlane32_swap(m, m, false, false);
  return pk_max_u16(p[0], p[1]);
}

struct MxGeom {
  const uint16_t *x;
  int64_t R, C, ld;
  uint32_t ntc_full;  // tile columns lying wholly inside the input
  uint32_t ntc;       // all tile columns
  uint32_t tr0;       // first tile row of the edge launch's bottom region
  uint32_t n_bottom;  // tiles of that region: (tile rows - tr0) * ntc
};

// Streaming stores of the encoded copies: written once and not read again by
// this kernel, so they bypass the cache's normal retention (measured 4 %
// faster on the 16384 x 2048 row+col case).
__device__ __forceinline__ void store_nt(uint2 *p, uint2 v) {
  typedef uint32_t u2v __attribute__((ext_vector_type(2)));
  __builtin_nontemporal_store(u2v{v.x, v.y}, reinterpret_cast<u2v *>(p));
}
__device__ __forceinline__ void store_nt(uint4 *p, uint4 v) {
  typedef uint32_t u4v __attribute__((ext_vector_type(4)));
  __builtin_nontemporal_store(u4v{v.x, v.y, v.z, v.w}, reinterpret_cast<u4v *>(p));
}

// Staging layout of one workgroup holding VT tiles (byte offsets in LDS).
template <int VT>
struct MxLds {
  static constexpr int QT = 0;                          // [128 cols][VT * 128 B]
  static constexpr int S = MX_T * MX_T * VT;            // [VT * 128 rows][4]
  static constexpr int ST = S + MX_T * 4 * VT;          // [VT * 4 row blocks][128 cols]
  static constexpr int BYTES = ST + MX_T * 4 * VT;
  // byte b (tile-block row) of staged column cl: the 16-byte chunks of a
  // staged column are XOR-swizzled by (cl / 8) % 8 in their low 3 index bits,
  // so that the 8-byte writes of the 16 column groups of a wave spread over
  // the LDS banks while a staged column still reads back in whole chunks
  static __device__ __forceinline__ int qt(int cl, int b) {
    return QT + cl * (MX_T * VT) + ((((b >> 4) ^ (cl >> 3)) & 7) << 4) + (b & ~127) + (b & 15);
  }
};

// Encode VT vertically adjacent tiles whose data is in v[k] and write both
// copies.  FULL: the tiles lie wholly inside the input, so no access needs a
// bounds test.
template <bool ROW, bool COL, bool FULL, int VT>
__device__ __forceinline__ void mx_tiles(const MxGeom &g, int64_t r0, int64_t c0,
                                         const uint4 (&v)[VT][8], uint8_t *__restrict__ lds,
                                         uint8_t *__restrict__ q, uint8_t *__restrict__ s,
                                         uint8_t *__restrict__ qT, uint8_t *__restrict__ sT) {
  using L = MxLds<VT>;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int c = lane & 15, r = lane >> 4;
  const int rl0 = 32 * wave + 8 * r;  // first of the lane's 8 rows in a tile
  const int64_t R = g.R, C = g.C;
  const int64_t col = c0 + 8 * c;

#pragma unroll
  for (int k = 0; k < VT; ++k) {
    const int rk = 128 * k + rl0;  // the lane's first row within the block
    // ---- row blocks: scale, encode, store; column maxima accumulate -------
    uint32_t cm[4] = {0, 0, 0, 0};  // column maxima, packed pairs 8c+2h, 8c+2h+1
    uint8_t *qrow = q + (r0 + rk) * C + col;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint4 w = v[k][i];
      const uint32_t a0 = w.x & 0x7FFF7FFFu, a1 = w.y & 0x7FFF7FFFu;
      const uint32_t a2 = w.z & 0x7FFF7FFFu, a3 = w.w & 0x7FFF7FFFu;
      if (COL) {
        cm[0] = pk_max_u16(cm[0], a0);
        cm[1] = pk_max_u16(cm[1], a1);
        cm[2] = pk_max_u16(cm[2], a2);
        cm[3] = pk_max_u16(cm[3], a3);
      }
      if (ROW) {
        const uint32_t m2 = pk_max_u16(pk_max_u16(a0, a1), pk_max_u16(a2, a3));
        const uint32_t m = max_xor2(max_xor1(max(m2 & 0xFFFFu, m2 >> 16)));
        const uint32_t sbits = mx_scale_bits_lo(m);
        const uint2 o = make_uint2(cvt4_e4m3_bf16_into(a0, w.x, w.y, sbits),
                                   cvt4_e4m3_bf16_into(a2, w.z, w.w, sbits));
        if (FULL || (col < C && r0 + rk + i < R))
          store_nt(reinterpret_cast<uint2 *>(qrow + i * C), o);
        // the 4 lanes of the block write the same byte
        lds[L::S + (rk + i) * 4 + (c >> 2)] = (uint8_t)(sbits >> 23);
      }
    }
    // ---- column blocks: 8 rows of column 8c + j here, 32 in the wave ------
    if (COL) {
#pragma unroll
      for (int h = 0; h < 4; ++h) cm[h] = pk_max_xor32(pk_max_xor16(cm[h]));
      uint2 sbs = make_uint2(0, 0);  // the 8 column scale bytes
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const uint32_t sbits = j & 1 ? mx_scale_bits_hi(cm[j >> 1]) : mx_scale_bits_lo(cm[j >> 1]);
        const uint32_t sel = j & 1 ? 0x07060302u : 0x05040100u;  // column j: rows i, i+1
        uint32_t p[4];
#pragma unroll
        for (int h = 0; h < 4; ++h)
          p[h] = __builtin_amdgcn_perm((&v[k][2 * h + 1].x)[j >> 1], (&v[k][2 * h].x)[j >> 1],
                                       sel);
        *reinterpret_cast<uint2 *>(lds + L::qt(8 * c + j, rk)) =
            make_uint2(cvt4_e4m3_bf16_into(p[0], p[0], p[1], sbits),
                       cvt4_e4m3_bf16_into(p[2], p[2], p[3], sbits));
        if (j < 4) sbs.x |= (sbits >> 23) << (8 * j);
        else sbs.y |= (sbits >> 23) << (8 * (j - 4));
      }
      // column scale bytes of this wave's 32-row block; the 4 lanes r = 0..3
      // write the same 8 bytes
      *reinterpret_cast<uint2 *>(lds + L::ST + (4 * k + wave) * MX_T + 8 * c) = sbs;
    }
  }
  __syncthreads();

  if (COL) {
    // transposed copy: staged column cl holds the block's VT * 128 rows
#pragma unroll
    for (int k = 0; k < 4 * VT; ++k) {
      const int ch = tid + 256 * k;  // 16-byte chunk: 8 * VT per staged column
      const int cl = ch / (8 * VT), b = (ch % (8 * VT)) * 16;
      const int64_t colg = c0 + cl, rowg = r0 + b;
      if (FULL || (colg < C && rowg < R))
        store_nt(reinterpret_cast<uint4 *>(qT + colg * R + rowg),
                 *reinterpret_cast<const uint4 *>(lds + L::qt(cl, b)));
    }
  }
  if (ROW && tid < MX_T * VT) {
    const int e = tid;  // block row
    if (FULL || r0 + e < R) {
      const uint32_t w4 = *reinterpret_cast<const uint32_t *>(lds + L::S + e * 4);
      uint8_t *dst = s + (r0 + e) * (C / 32) + c0 / 32;
      if ((C % 128) == 0) {
        *reinterpret_cast<uint32_t *>(dst) = w4;
      } else {
        for (int j = 0; j < 4 && c0 + 32 * j < C; ++j) dst[j] = (uint8_t)(w4 >> (8 * j));
      }
    }
  }
  if (COL && tid < MX_T) {
    const int e = tid;  // block column
    if (FULL || c0 + e < C) {
#pragma unroll
      for (int k = 0; k < VT; ++k) {
        const uint32_t w4 = (uint32_t)lds[L::ST + (4 * k) * MX_T + e] |
                            ((uint32_t)lds[L::ST + (4 * k + 1) * MX_T + e] << 8) |
                            ((uint32_t)lds[L::ST + (4 * k + 2) * MX_T + e] << 16) |
                            ((uint32_t)lds[L::ST + (4 * k + 3) * MX_T + e] << 24);
        const int64_t rt = r0 + 128 * k;
        if (!FULL && rt >= R) break;
        uint8_t *dst = sT + (c0 + e) * (R / 32) + rt / 32;
        if ((R % 128) == 0) {
          *reinterpret_cast<uint32_t *>(dst) = w4;
        } else {
          for (int j = 0; j < 4 && rt + 32 * j < R; ++j) dst[j] = (uint8_t)(w4 >> (8 * j));
        }
      }
    }
  }
}

// FULL launch: workgroup b takes block b of VT x 128 rows by 128 columns in
// row-major block order.  Edge launch (VT = 1): tile b of the bottom region
// (tile rows tr0 .. end, all tile columns), then of the right column of
// partial tiles beside the full bands.
template <bool ROW, bool COL, bool FULL, int VT>
__global__ __launch_bounds__(256) void k_quantize_mxfp8(MxGeom g, uint8_t *__restrict__ q,
                                                       uint8_t *__restrict__ s,
                                                       uint8_t *__restrict__ qT,
                                                       uint8_t *__restrict__ sT) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[MxLds<VT>::BYTES];
  const uint32_t b = blockIdx.x;
  uint32_t tr, tc;
  if (FULL) {
    tr = (b / g.ntc_full) * VT;
    tc = b % g.ntc_full;
  } else if (b < g.n_bottom) {
    tr = g.tr0 + b / g.ntc;
    tc = b % g.ntc;
  } else {
    tr = b - g.n_bottom;
    tc = g.ntc_full;
  }
  const int64_t r0 = (int64_t)tr * MX_T, c0 = (int64_t)tc * MX_T;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int c = lane & 15, rl0 = 32 * wave + 8 * (lane >> 4);
  const int64_t col = c0 + 8 * c;
  const uint16_t *p = g.x + (r0 + rl0) * g.ld + col;
  uint4 v[VT][8];
#pragma unroll
  for (int k = 0; k < VT; ++k) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint16_t *src = p + (128 * k + i) * g.ld;
      if (FULL) {
        v[k][i] = *reinterpret_cast<const uint4 *>(src);
      } else {
        v[k][i] = make_uint4(0, 0, 0, 0);
        if (col < g.C && r0 + 128 * k + rl0 + i < g.R) v[k][i] = *reinterpret_cast<const uint4 *>(src);
      }
    }
  }
  mx_tiles<ROW, COL, FULL, VT>(g, r0, c0, v, lds, q, s, qT, sT);
}

// Tiles per interior workgroup.  On MI355X (16384 x 2048 input) one tile per
// workgroup measured 30.2 us against 32.8 us for pairs: the larger per-
// workgroup footprint costs more in the memory system than the overlap of the
// second tile's loads gains.
constexpr int MX_VT = 1;

template <bool ROW, bool COL>
static void launch_mx(const MxGeom &g, uint32_t n_full, uint32_t n_edge, uint8_t *q, uint8_t *s,
                      uint8_t *qT, uint8_t *sT, hipStream_t st) {
  if (n_full)
    hipLaunchKernelGGL((k_quantize_mxfp8<ROW, COL, true, MX_VT>), dim3(n_full), dim3(256), 0, st,
                       g, q, s, qT, sT);
  if (n_edge)
    hipLaunchKernelGGL((k_quantize_mxfp8<ROW, COL, false, 1>), dim3(n_edge), dim3(256), 0, st, g,
                       q, s, qT, sT);
}

hipError_t launch_quantize_mxfp8(const uint16_t *x, int64_t R, int64_t C, int64_t ld,
                                 uint8_t *q, uint8_t *s, uint8_t *qT, uint8_t *sT,
                                 hipStream_t st) {
  if (R == 0 || C == 0) return hipSuccess;
  const int64_t ntc_full = C / MX_T, ntr_full = R / MX_T;
  const int64_t ntc = (C + MX_T - 1) / MX_T, ntr = (R + MX_T - 1) / MX_T;
  if (ntc * ntr >= (int64_t)1 << 31) return hipErrorInvalidValue;
  const int64_t nblk_rows = ntr_full / MX_VT;  // interior blocks of VT tile rows
  const int64_t tr0 = nblk_rows * MX_VT;
  MxGeom g{x, R, C, ld, (uint32_t)ntc_full, (uint32_t)ntc, (uint32_t)tr0,
           (uint32_t)((ntr - tr0) * ntc)};
  const uint32_t n_full = (uint32_t)(nblk_rows * ntc_full);
  const uint32_t n_edge = g.n_bottom + (uint32_t)(C % MX_T ? tr0 : 0);
  const bool row = q != nullptr, col = qT != nullptr;
  if (row && col) launch_mx<true, true>(g, n_full, n_edge, q, s, qT, sT, st);
  else if (row) launch_mx<true, false>(g, n_full, n_edge, q, s, qT, sT, st);
  else launch_mx<false, true>(g, n_full, n_edge, q, s, qT, sT, st);
  return hipGetLastError();
}

}  // namespace pqm
