// grouped_gemm.hip -- grouped GEMM over routed experts on gfx950 MFMA.
//
// "miniTE technical report", 5.2: the quantized rows of all experts sit in
// one contiguous buffer with offsets marking the expert boundaries and are
// handed to one dense grouped GEMM; metadata stays on the device and empty
// experts are handled inside.  Here one launch covers every expert: each
// workgroup reads the offsets, derives its (expert, row tile, column tile)
// on the device and skips nothing on the host (no per-expert host work).
// 5.4: the accumulator is scaled in binary32 (ACC = block-scaled GEMM;
// ACC *= alpha).
//
// MXFP8: v_mfma_scale_f32_32x32x64_f8f6f4 consumes E4M3 operands with one
// E8M0 scale per 32 K-values per row, which is the MXFP8 block layout, so
// the scales go to the matrix core unchanged.  K % 128 == 0 runs the
// pipelined 256 x 256 kernel (k_gemm_mxfp8_q: eight waves, 128-byte ring
// steps, an expert's last tile of at most 128 rows as 128 x 256); other K
// the simpler 128 x 128 kernel with register-staged tiles.  Lane layout (verified on the
// hardware): a lane holds row (lane % 32); its bytes 0-15 are K
// 16*(lane/32) .. +15 of the first 32-block and bytes 16-31 the same offsets
// in the second block; lane 32*b + r supplies the scale of row r, block b.
// The 32x32 fp32 accumulator of lane l holds column l % 32, rows
// 8*(i/4) + 4*(l/32) + i%4 for i = 0..15.
//
// BF16 (backward on dequantized or original operands): v_mfma_f32_32x32x16
// with 8 consecutive K per lane (lanes 32..63 hold K 8..15).  Operands whose
// contraction index is not contiguous in memory (dgrad's weight, both wgrad
// operands) are transposed while they are staged into LDS.
#include "nvfp4_encode.hpp"
#include "pqm_device.hpp"
#include "pqm_internal.hpp"

namespace pqm {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));

constexpr int GT_M = 128;   // workgroup tile rows
constexpr int GT_N = 128;   // workgroup tile columns
constexpr int GT_KB = 128;  // K bytes staged per step (128 fp8 or 64 bf16)
constexpr int GT_PITCH = GT_KB + 16;  // LDS row pitch, bytes (bank spread)

struct TileInfo {
  int64_t g, row0, row_end, n0;
};

// Workgroup tile lookup for the row-tiled kinds (FPROP / DGRAD).  Logical
// tile T enumerates (global row tile, column tile) with columns fastest;
// global row tiles enumerate experts in order, ceil(M_g / GT_M) each.  The
// hardware places workgroup b on XCD b % 8; b is remapped so that each XCD
// owns a contiguous range of logical tiles (the tiles of one expert share
// its weight slices in that XCD's L2).  Returns false if no tile.
template <int TN = GT_N, int TM = GT_M>
__device__ bool lookup_row_tile(const int64_t *__restrict__ offsets, int64_t G, int64_t ntn,
                                TileInfo &ti, int64_t *sh) {
  const int lane = threadIdx.x & 63;
  constexpr int NC = 8;  // up to 64 NC groups: all offsets in one round of loads
  if (threadIdx.x < 64 && G <= 64 * NC) {
    int64_t lo[NC], hi[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) {  // clamped, so every load is in bounds
      const int64_t g = min((int64_t)(64 * c + lane), G);
      lo[c] = offsets[g];
      hi[c] = offsets[min(g + 1, G)];
    }
    const int nch = (int)((G + 63) / 64);
    int cnt[NC], total = 0;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      cnt[c] = 64 * c + lane < G ? (int)((hi[c] - lo[c] + TM - 1) / TM) : 0;
      if (c < nch) {
        int t = cnt[c];
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) t += __shfl_xor(t, o, 64);
        total += t;
      }
    }
    const int64_t real = (int64_t)total * ntn;
    const int64_t per_xcd = (real + 7) / 8;
    const int64_t b = blockIdx.x;
    const int64_t T = (b % 8) * per_xcd + b / 8;
    int64_t found_g = -1, row0 = 0, row_end = 0;
    if (b < 8 * per_xcd && T < real) {
      const int mt = (int)(T / ntn);
      int base = 0;
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        if (c >= nch || found_g >= 0) break;
        int incl = cnt[c];
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
          const int t = __shfl_up(incl, o, 64);
          if (lane >= o) incl += t;
        }
        const bool hit = cnt[c] > 0 && mt >= base + incl - cnt[c] && mt < base + incl;
        const unsigned long long m = __ballot(hit);
        if (m) {
          const int src = __ffsll((long long)m) - 1;
          found_g = 64 * c + src;
          row0 = __shfl(lo[c], src, 64) +
                 (int64_t)(mt - base - __shfl(incl - cnt[c], src, 64)) * TM;
          row_end = __shfl(hi[c], src, 64);
        }
        base += __shfl(incl, 63, 64);
      }
      if (lane == 0) {
        sh[0] = found_g;
        sh[1] = row0;
        sh[2] = row_end;
        sh[3] = (T % ntn) * TN;
      }
    } else if (lane == 0) {
      sh[0] = -1;
    }
  } else if (threadIdx.x < 64) {
    // pass 1: total row tiles
    int64_t total = 0;
    for (int64_t c0 = 0; c0 < G; c0 += 64) {
      const int64_t g = c0 + lane;
      int64_t cnt = 0;
      if (g < G) cnt = (offsets[g + 1] - offsets[g] + TM - 1) / TM;
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) cnt += __shfl_xor(cnt, o, 64);
      total += cnt;
    }
    const int64_t real = total * ntn;
    const int64_t per_xcd = (real + 7) / 8;
    const int64_t b = blockIdx.x;
    const int64_t T = (b % 8) * per_xcd + b / 8;
    int64_t found_g = -1, row0 = 0, row_end = 0;
    if (b < 8 * per_xcd && T < real) {
      const int64_t mt = T / ntn;
      int64_t base = 0;
      for (int64_t c0 = 0; c0 < G && found_g < 0; c0 += 64) {
        const int64_t g = c0 + lane;
        int64_t lo = 0, hi = 0, cnt = 0;
        if (g < G) {
          lo = offsets[g];
          hi = offsets[g + 1];
          cnt = (hi - lo + TM - 1) / TM;
        }
        int64_t incl = cnt;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
          const int64_t t = __shfl_up(incl, o, 64);
          if (lane >= o) incl += t;
        }
        const bool hit = g < G && mt >= base + incl - cnt && mt < base + incl;
        const unsigned long long m = __ballot(hit);
        if (m) {
          const int src = __ffsll((long long)m) - 1;
          const int64_t gg = __shfl(g, src, 64);
          const int64_t l0 = __shfl(lo, src, 64);
          const int64_t h0 = __shfl(hi, src, 64);
          const int64_t ex = __shfl(incl - cnt, src, 64);
          found_g = gg;
          row0 = l0 + (mt - base - ex) * TM;
          row_end = h0;
        }
        base += __shfl(incl, 63, 64);
      }
      if (lane == 0) {
        sh[0] = found_g;
        sh[1] = row0;
        sh[2] = row_end;
        sh[3] = (T % ntn) * TN;
      }
    } else if (lane == 0) {
      sh[0] = -1;
    }
  }
  __syncthreads();
  ti.g = sh[0];
  ti.row0 = sh[1];
  ti.row_end = sh[2];
  ti.n0 = sh[3];
  return ti.g >= 0;
}

// Stage a 128-row x 128-byte operand tile whose K is contiguous in memory:
// 4 x 16-byte loads per lane, rows beyond `rows` or K bytes beyond `kbytes`
// read as zero.
struct KContigLoader {
  uint4 v[4];
  __device__ void load(const uint8_t *__restrict__ base, int64_t row_stride, int64_t rows,
                       int64_t k0_bytes, int64_t kbytes) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = threadIdx.x + 256 * i;
      const int r = c >> 3, cc = (c & 7) * 16;
      v[i] = make_uint4(0, 0, 0, 0);
      if (r < rows && k0_bytes + cc < kbytes)
        v[i] = *reinterpret_cast<const uint4 *>(base + r * row_stride + k0_bytes + cc);
    }
  }
  __device__ void store(uint8_t *lds) const {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = threadIdx.x + 256 * i;
      *reinterpret_cast<uint4 *>(lds + (c >> 3) * GT_PITCH + (c & 7) * 16) = v[i];
    }
  }
};

__device__ __forceinline__ v8i frag_fp8(const uint8_t *lds, int row, int s) {
  const int lane = threadIdx.x & 63;
  const uint8_t *p = lds + row * GT_PITCH + 64 * s + 16 * (lane >> 5);
  const uint4 lo = *reinterpret_cast<const uint4 *>(p);
  const uint4 hi = *reinterpret_cast<const uint4 *>(p + 32);
  v8i r;
  r[0] = lo.x; r[1] = lo.y; r[2] = lo.z; r[3] = lo.w;
  r[4] = hi.x; r[5] = hi.y; r[6] = hi.z; r[7] = hi.w;
  return r;
}

// Write one 32x32 accumulator tile (rows row0 + rbase .., cols n0 + cbase ..),
// optionally scaled in binary32 by alpha_row[row] and alpha_col(col), plus
// bias[col] (the expert's bias row, binary32) when given, rounded once.
template <bool OUT_F32>
__device__ __forceinline__ void store_acc(const v16f &acc, void *out, int64_t ldo, int64_t row0,
                                          int64_t row_end, int64_t n0, int64_t N, int rbase,
                                          int cbase, const float *alpha_row = nullptr,
                                          float alpha_col = 1.0f, const float *bias = nullptr) {
  const int lane = threadIdx.x & 63;
  const int64_t col = n0 + cbase + (lane & 31);
  if (col >= N) return;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int64_t row = row0 + rbase + 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
    if (row < row_end) {
      float v = acc[i];
      // alpha_a * alpha_b is exact in binary64; one scaling of the
      // accumulator avoids an intermediate binary32 overflow (a bf16-max
      // token has alpha_a near 2^116)
      if (alpha_row) {
        const double sv = (double)v * ((double)alpha_row[row] * (double)alpha_col);
        v = (float)(bias ? sv + (double)bias[col] : sv);
      } else if (bias) {
        v += bias[col];
      }
      if (OUT_F32)
        static_cast<float *>(out)[row * ldo + col] = v;
      else
        static_cast<uint16_t *>(out)[row * ldo + col] = (uint16_t)f32_to_bf16_rne(v);
    }
  }
}

// ------------------------------------------------------------------ MXFP8

template <bool OUT_F32>
__global__ __launch_bounds__(256) void k_gemm_mxfp8(
    const uint8_t *__restrict__ A, const uint8_t *__restrict__ As,
    const uint8_t *__restrict__ B, const uint8_t *__restrict__ Bs,
    const int64_t *__restrict__ offsets, int64_t G, int64_t N, int64_t K, int64_t ntn,
    void *__restrict__ out, const float *__restrict__ bias) {
  __shared__ __attribute__((aligned(16))) uint8_t lA[GT_M * GT_PITCH];
  __shared__ __attribute__((aligned(16))) uint8_t lB[GT_N * GT_PITCH];
  __shared__ int64_t sh[4];
  TileInfo ti;
  if (!lookup_row_tile(offsets, G, ntn, ti, sh)) return;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int64_t KS = K / 32;  // scale bytes per row
  const int64_t rows_a = ti.row_end - ti.row0;
  const int64_t rows_b = N - ti.n0;
  const uint8_t *Ab = A + ti.row0 * K;
  const uint8_t *Bb = B + (ti.g * N + ti.n0) * K;
  const uint8_t *Asb = As + ti.row0 * KS;
  const uint8_t *Bsb = Bs + (ti.g * N + ti.n0) * KS;

  v16f acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  KContigLoader la, lb;
  la.load(Ab, K, rows_a, 0, K);
  lb.load(Bb, K, rows_b, 0, K);
  const int nk = (int)((K + GT_KB - 1) / GT_KB);
  for (int kt = 0; kt < nk; ++kt) {
    la.store(lA);
    lb.store(lB);
    __syncthreads();
    if (kt + 1 < nk) {
      la.load(Ab, K, rows_a, (int64_t)(kt + 1) * GT_KB, K);
      lb.load(Bb, K, rows_b, (int64_t)(kt + 1) * GT_KB, K);
    }
    // scales: lane supplies block (kt*4 + 2s + lane/32) of its row
    int sa[2][2], sbv[2][2];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const int64_t kb = (int64_t)kt * 4 + 2 * s + (lane >> 5);
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int ra = wm * 64 + 32 * i + (lane & 31);
        sa[i][s] = (ra < rows_a && kb < KS) ? Asb[ra * KS + kb] : 127;
        const int rb = wn * 64 + 32 * i + (lane & 31);
        sbv[i][s] = (rb < rows_b && kb < KS) ? Bsb[rb * KS + kb] : 127;
      }
    }
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      v8i fa[2], fb[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        fa[i] = frag_fp8(lA, wm * 64 + 32 * i + (lane & 31), s);
        fb[i] = frag_fp8(lB, wn * 64 + 32 * i + (lane & 31), s);
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
              fa[i], fb[j], acc[i][j], 0, 0, 0, sa[i][s], 0, sbv[j][s]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
      store_acc<OUT_F32>(acc[i][j], out, N, ti.row0, ti.row_end, ti.n0, N, wm * 64 + 32 * i,
                         wn * 64 + 32 * j, nullptr, 1.0f, bias ? bias + ti.g * N : nullptr);
}

// ------------------------------------------------- MXFP8, pipelined large tiles
//
// Workgroup tile TM rows x 256 columns (TM = 256 or 128), one workgroup of
// 4 waves per CU; wave (wm, wn) owns rows TM/2 wm .. and columns 128 wn ..
// as FI x 4 accumulators of 32 x 32 in AGPRs (FI = TM / 64).  Per 64-K step
// and wave, 2 (FI + 4) fragment reads feed 4 FI MFMAs: with TM = 256 a wave
// reads 8 KB of LDS for 16 MFMAs, half the traffic per flop of TM = 128.
//
// Operands reach LDS by direct global->LDS loads (global_load_lds_dwordx4:
// lane l's 16 bytes land at M0 + 16 l), issued from inline assembly so that
// the compiler does not serialise them against the LDS reads of other ring
// slots; the code waits for them explicitly.  The ring has 3 slots of one
// 64-K step each.  During step k a wave multiplies operands it read from
// LDS during step k-1, reads step k+1's operands and requests step k+3 into
// the slot step k came from.  Before step k it waits until only its loads of
// step k+2 are pending (and its LDS reads are done) and meets the other
// waves at a barrier, which publishes step k+1 and frees slot k % 3.  Past
// the last step the requests repeat the last step (in bounds, never read)
// and reads take stale slots, so the loop has no branches; the kernel drains
// its loads before it exits.  Rows of a slot are 64 bytes whose 16-byte
// chunks are XOR-swizzled by (row / 4) % 4; the swizzle goes into the global
// addresses.  All scale bytes of the tile's rows are loaded once, in groups
// of 16 rows.  Rows past
// the expert's end (A) or past N (B) load a clamped valid row; their results
// are never stored.  Requires K % 128 == 0 and K / 32 <= MAX_KS.
template <int TM>
struct Mx3 {
  static constexpr int TN = 256;                  // workgroup tile columns
  static constexpr int ROWS = TM + TN;            // staged rows per step
  static constexpr int SLOT = ROWS * 64;          // bytes per ring slot
  static constexpr int NSLOT = 3;
  static constexpr int MAX_KS = TM == 256 ? 64 : 96;  // scale bytes per row
  static constexpr int LDS = NSLOT * SLOT + ROWS * MAX_KS;
  static constexpr int CA = TM / 64, CB = TN / 64;    // 16-byte chunks per lane per step
  static constexpr int OPS = CA + CB;                 // loads per lane per step
  static constexpr int FI = TM / 64, FJ = 4;          // fragments per wave
};

#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
// 16 bytes per lane from global `src` into LDS at m0 + 16 * lane.
__device__ __forceinline__ void dma16(const void *src, uint32_t m0) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src), "s"(m0)
               : "memory", "m0");
}
// 4 bytes per lane from global `src` into LDS at m0 + 4 * lane.
__device__ __forceinline__ void dma4(const void *src, uint32_t m0) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dword %0, off" ::"v"(src), "s"(m0)
               : "memory", "m0");
}
#pragma clang diagnostic pop

template <int n>
__device__ __forceinline__ void vm_wait() {
  static_assert(n >= 0 && n < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((n & 0xF) | ((n >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}
__device__ __forceinline__ void lgkm_wait0() { __builtin_amdgcn_s_waitcnt(0xC07F); }

// Workgroup barrier that no LDS access moves across in the compiler (for
// plain LDS stores and loads next to it; the caller waits for its own LDS and
// DMA accesses first).
__device__ __forceinline__ void wg_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

__device__ __forceinline__ uint32_t lds_addr(const void *p) {
  return (uint32_t)(uintptr_t)p;
}

template <int TM>
struct Mx3Src {
  const uint8_t *Ab, *Bb;                    // tile bases
  uint32_t oa[Mx3<TM>::CA], ob[Mx3<TM>::CB];  // per-lane sources of a step's chunks (step 0)
  uint32_t dst;                              // LDS address of slot 0, this wave's chunks
};

// Request step kt into slot `slot`.
template <int TM>
__device__ __forceinline__ void mx3_issue(const Mx3Src<TM> &L, int kt, int slot) {
  using C = Mx3<TM>;
  const uint32_t kb = (uint32_t)kt * 64u;
  const uint32_t base = L.dst + (uint32_t)slot * C::SLOT;
#pragma unroll
  for (int i = 0; i < C::CA; ++i) dma16(L.Ab + (L.oa[i] + kb), base + i * 4096);
#pragma unroll
  for (int i = 0; i < C::CB; ++i) dma16(L.Bb + (L.ob[i] + kb), base + TM * 64 + i * 4096);
}

// Byte offset of 16-byte chunk `chunk` of row `row` in a ring slot.
__device__ __forceinline__ int mx3_off(int row, int chunk) {
  return row * 64 + ((chunk ^ (row >> 2)) & 3) * 16;
}

// A wave's operands of one 64-K step and their scale bytes.
template <int TM>
struct Mx3Frags {
  v8i a[Mx3<TM>::FI], b[Mx3<TM>::FJ];
  int sa[Mx3<TM>::FI], sb[Mx3<TM>::FJ];
};

// Per-lane LDS offsets of the operands within a slot (fragment f of a row
// group sits 2048 f bytes after fragment 0: rows 32 apart share the swizzle)
// and of the scale bytes (16-row groups, dword-major within a group).
struct Mx3Lane {
  int a_lo, a_hi, b_lo, b_hi;  // chunks h and 2 + h of the first A / B row
  int sa, sb;                  // first scale byte of the first A / B row
  int ks;                      // scale bytes per row
};

template <int TM>
__device__ __forceinline__ void mx3_read(const uint8_t *lds, int kt, int slot, const Mx3Lane &o,
                                         Mx3Frags<TM> &F) {
  using C = Mx3<TM>;
  const uint8_t *cur = lds + slot * C::SLOT;
  const int blk = 2 * kt + ((threadIdx.x & 63) >> 5);
  const uint8_t *sc = lds + C::NSLOT * C::SLOT + (blk >> 2) * 64 + (blk & 3);
#pragma unroll
  for (int i = 0; i < C::FI; ++i) {
    const uint4 lo = *reinterpret_cast<const uint4 *>(cur + o.a_lo + 2048 * i);
    const uint4 hi = *reinterpret_cast<const uint4 *>(cur + o.a_hi + 2048 * i);
    F.a[i] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
    F.sa[i] = sc[o.sa + 2 * i * o.ks * 16];
  }
#pragma unroll
  for (int j = 0; j < C::FJ; ++j) {
    const uint4 lo = *reinterpret_cast<const uint4 *>(cur + o.b_lo + 2048 * j);
    const uint4 hi = *reinterpret_cast<const uint4 *>(cur + o.b_hi + 2048 * j);
    F.b[j] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
    F.sb[j] = sc[o.sb + 2 * j * o.ks * 16];
  }
}

// Lane (h, r) holds a and b; one swap of the upper half-wave's a with the
// lower half-wave's b leaves lane (0, r) with lo = its a, hi = lane (1, r)'s
// a, and lane (1, r) with lo = lane (0, r)'s b, hi = its b.  (Rows r of a
// 32 x 32 fragment: a, b the runs of 4 columns at 8 g + 4 h and 8 g + 8 +
// 4 h give each lane 8 consecutive columns.)
__device__ __forceinline__ void half_trade(float a, float b, float &lo, float &hi) {
  const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false,
                                                   false);
  lo = __uint_as_float(sw[0]);
  hi = __uint_as_float(sw[1]);
}

// The weight fragment is the MFMA's first operand, the token fragment its
// second, so each accumulator holds a transposed 32 x 32 tile: lane l owns
// token row l % 32 and output columns 8 g + 4 (l / 32) + 0..3 (g = 0..3),
// four runs of 4 consecutive columns.
// Write one transposed accumulator (token rows row0 + rbase + 0..31, output
// columns n0 + cbase + 0..31).  Lane l holds columns 8 g + 4 (l / 32) + 0..3
// of its row.  binary32: one 16-byte store per run, so the two lanes of a
// row fill a whole 32-byte sector per instruction.  bf16: the gfx950 lane
// swap between lanes l and l + 32 trades run g = 1 (3) of the low half for
// run 0 (2) of the high half, after which lane l holds columns
// 16 p + 8 (l / 32) + 0..7, p = 0, 1: two 16-byte stores per lane.
// bias: the expert's bias row (binary32, N columns) added to every value
// before the output rounding, or null.
template <bool OUT_F32>
__device__ __forceinline__ void mx3_store(const v16f &acc, void *out, int64_t N, int64_t row0,
                                          int64_t row_end, int64_t n0, int rbase, int cbase,
                                          const float *bias = nullptr) {
  const int lane = threadIdx.x & 63, h = lane >> 5;
  const int64_t row = row0 + rbase + (lane & 31);
  if (OUT_F32) {
    // run g = registers 4 g .. 4 g + 3 = columns 8 g + 4 h + 0..3
    if (row >= row_end) return;
    float *orow = static_cast<float *>(out) + row * N;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int64_t col = n0 + cbase + 8 * g + 4 * h;
      float v[4] = {acc[4 * g], acc[4 * g + 1], acc[4 * g + 2], acc[4 * g + 3]};
      if (bias) {
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] += bias[min(col + e, N - 1)];
      }
      if ((N & 3) == 0 && col + 3 < N) {
        *reinterpret_cast<float4 *>(orow + col) = make_float4(v[0], v[1], v[2], v[3]);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (col + e < N) orow[col + e] = v[e];
      }
    }
    return;
  }
  const bool vec = (N & 7) == 0;
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    // runs 2p (own) and 2p+1 (own); the low half keeps run 2p and receives
    // the high half's run 2p, the high half keeps run 2p+1 and receives the
    // low half's run 2p+1
    float lo[4], hi[4];  // this lane's first and second 4 columns after the swap
#pragma unroll
    for (int e = 0; e < 4; ++e) half_trade(acc[8 * p + e], acc[8 * p + 4 + e], lo[e], hi[e]);
    const int64_t col = n0 + cbase + 16 * p + 8 * h;
    if (row >= row_end) continue;
    if (bias) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        lo[e] += bias[min(col + e, N - 1)];
        hi[e] += bias[min(col + 4 + e, N - 1)];
      }
    }
    if (vec && col + 7 < N) {
      // hardware pair conversion (nearest even, as f32_to_bf16_rne)
      const uint4 w = make_uint4(pk_bf16_rne(lo[0], lo[1]), pk_bf16_rne(lo[2], lo[3]),
                                 pk_bf16_rne(hi[0], hi[1]), pk_bf16_rne(hi[2], hi[3]));
      *reinterpret_cast<uint4 *>(static_cast<uint16_t *>(out) + row * N + col) = w;
    } else {
      const float v[8] = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (col + e < N)
          static_cast<uint16_t *>(out)[row * N + col + e] = (uint16_t)f32_to_bf16_rne(v[e]);
    }
  }
}

// Step kt from slot `slot`: operands in `cur` (read during the previous
// step).  Publish step kt+1, refill `slot` with step kt+3, read step kt+1's
// operands into `next`, multiply `cur`.  src(q, kb) gives the global source
// of refill load q (A chunks 0 .. CA-1, then B chunks) at step byte kb.
template <int TM, class Src>
__device__ __forceinline__ void mx3_step_with(const Mx3Src<TM> &L, const uint8_t *lds,
                                              const Mx3Lane &o, int kt, int nk, int slot,
                                              v16f (&acc)[Mx3<TM>::FI][Mx3<TM>::FJ],
                                              const Mx3Frags<TM> &cur, Mx3Frags<TM> &next,
                                              const Src &src) {
  using C = Mx3<TM>;
  vm_wait<C::OPS>();  // own loads of step kt+1 done; step kt+2 may be pending
  lgkm_wait0();       // own reads of `slot` done before it is refilled
  __builtin_amdgcn_s_barrier();
  // One wave per SIMD: while an MFMA occupies the matrix core (64 cycles) the
  // wave can issue other instructions, but the next MFMA waits.  So each
  // MFMA is followed by a slice of the step's other work: two of the refill
  // loads of step kt+3, then one fragment's operand reads of step kt+1.
  const uint8_t *rd = lds + (slot == 2 ? 0 : slot + 1) * C::SLOT;
  const uint32_t kb = (uint32_t)min(kt + 3, nk - 1) * 64u;
  const uint32_t base = L.dst + (uint32_t)slot * C::SLOT;
  const int blk = 2 * (kt + 1) + ((threadIdx.x & 63) >> 5);
  const uint8_t *sc = lds + C::NSLOT * C::SLOT + (blk >> 2) * 64 + (blk & 3);
  constexpr int NL = C::CA + C::CB, ND = (NL + 1) / 2;  // loads, MFMAs carrying them
#pragma unroll
  for (int m = 0; m < C::FI * C::FJ; ++m) {
    const int j = m / C::FI, i = m % C::FI;
    acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(cur.b[j], cur.a[i], acc[i][j], 0,
                                                                 0, 0, cur.sb[j], 0, cur.sa[i]);
    if (m < ND) {
#pragma unroll
      for (int q = 2 * m; q < 2 * m + 2 && q < NL; ++q) {
        dma16(src(q, kb), base + (q < C::CA ? q * 4096 : TM * 64 + (q - C::CA) * 4096));
      }
    } else if (m - ND < C::FI) {
      const int f = m - ND;
      const uint4 lo = *reinterpret_cast<const uint4 *>(rd + o.a_lo + 2048 * f);
      const uint4 hi = *reinterpret_cast<const uint4 *>(rd + o.a_hi + 2048 * f);
      next.a[f] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
      next.sa[f] = sc[o.sa + 2 * f * o.ks * 16];
    } else if (m - ND - C::FI < C::FJ) {
      const int f = m - ND - C::FI;
      const uint4 lo = *reinterpret_cast<const uint4 *>(rd + o.b_lo + 2048 * f);
      const uint4 hi = *reinterpret_cast<const uint4 *>(rd + o.b_hi + 2048 * f);
      next.b[f] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
      next.sb[f] = sc[o.sb + 2 * f * o.ks * 16];
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  // fragments left over when there are fewer MFMAs than slices (TM = 128)
#pragma unroll
  for (int f = C::FI * C::FJ - ND; f < C::FI + C::FJ; ++f) {
    if (f < C::FI) {
      const uint4 lo = *reinterpret_cast<const uint4 *>(rd + o.a_lo + 2048 * f);
      const uint4 hi = *reinterpret_cast<const uint4 *>(rd + o.a_hi + 2048 * f);
      next.a[f] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
      next.sa[f] = sc[o.sa + 2 * f * o.ks * 16];
    } else {
      const int g = f - C::FI;
      const uint4 lo = *reinterpret_cast<const uint4 *>(rd + o.b_lo + 2048 * g);
      const uint4 hi = *reinterpret_cast<const uint4 *>(rd + o.b_hi + 2048 * g);
      next.b[g] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
      next.sb[g] = sc[o.sb + 2 * g * o.ks * 16];
    }
  }
}

template <int TM>
__device__ __forceinline__ void mx3_step(const Mx3Src<TM> &L, const uint8_t *lds,
                                         const Mx3Lane &o, int kt, int nk, int slot,
                                         v16f (&acc)[Mx3<TM>::FI][Mx3<TM>::FJ],
                                         const Mx3Frags<TM> &cur, Mx3Frags<TM> &next) {
  mx3_step_with<TM>(L, lds, o, kt, nk, slot, acc, cur, next, [&](int q, uint32_t kb) {
    return q < Mx3<TM>::CA ? L.Ab + (L.oa[q] + kb) : L.Bb + (L.ob[q - Mx3<TM>::CA] + kb);
  });
}

// Fused gate_up epilogue (SwiGLU x prob, then the row-wise MXFP8 encoding
// of D, the FC2 operand).  The gate_up weight W_g [2I, K] is read with its
// rows permuted per 256-column tile tn so that every lane finds matching
// gate and up columns in its own accumulator registers: a transposed 32 x 32
// accumulator gives lane h * 32 + r the columns 8 g + 4 h + e (g, e = 0..3)
// of its fragment as registers 4 g + e, and tile column
// c = 128 wn + 32 j + 8 g + 4 h + e is made gate (g even) or up (g odd) of
//   dcol = 128 tn + 64 wn + 32 (j / 2) + 16 h + 8 (j % 2) + 4 (g / 2) + e,
// i.e. W row dcol or I + dcol.  A lane half then holds 16 consecutive D
// columns of each 32-column block (fragments j, j + 1).
struct SwigluEpi {
  const float *prob;    // router probability, indexed by src[row] (or row)
  const int32_t *src;
  int64_t I;            // D columns; I % 128 == 0
  uint8_t *q, *s;       // D in MXFP8: q [M, I] E4M3, s [M, I / 32] E8M0
};

__device__ __forceinline__ int64_t swiglu_w_row(int c, int64_t tn, int64_t I) {
  const int wn = c >> 7, j = (c >> 5) & 3, g = (c >> 3) & 3, hh = (c >> 2) & 1, e = c & 3;
  const int64_t dcol =
      128 * tn + 64 * wn + 32 * (j >> 1) + 16 * hh + 8 * (j & 1) + 4 * (g >> 1) + e;
  return (g & 1) ? I + dcol : dcol;
}

// D for one fragment-pair block of one wave: acc[i][2 jj], acc[i][2 jj + 1]
// (token rows row0 + rbase + 0..31, D columns dbase + 0..31).
__device__ __forceinline__ void swiglu_store(const v16f &a0, const v16f &a1,
                                             const SwigluEpi &ep, int64_t row0, int64_t row_end,
                                             int rbase, int64_t dbase) {
  const int lane = threadIdx.x & 63, h = lane >> 5;
  const int64_t row = row0 + rbase + (lane & 31);
  const bool ok = row < row_end;
  const float pr = ok ? ep.prob[ep.src ? ep.src[row] : row] : 0.0f;
  uint32_t dw[8];  // 16 D values (bf16 pairs): columns dbase + 16 h + 0..15
#pragma unroll
  for (int jo = 0; jo < 2; ++jo) {
    const v16f &acc = jo ? a1 : a0;
#pragma unroll
    for (int gp = 0; gp < 2; ++gp)
#pragma unroll
      for (int e2 = 0; e2 < 2; ++e2) {
        // gate (register 8 gp + e) and up (8 gp + 4 + e) of D column
        // 8 jo + 4 gp + e, rounded to bf16 as the GEMM's output would be,
        // then the weighted SwiGLU exactly as pqm_swiglu_prob computes it
        const int e = 2 * e2;
        const uint32_t gw = pk_bf16_rne(acc[8 * gp + e], acc[8 * gp + e + 1]);
        const uint32_t uw = pk_bf16_rne(acc[8 * gp + 4 + e], acc[8 * gp + 4 + e + 1]);
        dw[4 * jo + 2 * gp + e2] =
            pk_bf16_rne(swiglu_f32(bf16_lo_f32(gw), bf16_lo_f32(uw), pr),
                        swiglu_f32(bf16_hi_f32(gw), bf16_hi_f32(uw), pr));
      }
  }
  // block maximum over the 32 D columns: this lane's 16, then the other half
  uint32_t mm = 0;
#pragma unroll
  for (int k = 0; k < 8; ++k) mm = pk_max_u16(mm, dw[k] & 0x7FFF7FFFu);
  mm = max(mm & 0xFFFFu, mm >> 16);
  {
    const auto sw = __builtin_amdgcn_permlane32_swap(mm, mm, false, false);
    mm = max(sw[0], sw[1]);
  }
  const uint32_t b = mx_scale_byte(mm);
  const float scale = __uint_as_float(b << 23);
  if (ok) {
    const uint4 qv = make_uint4(cvt4_e4m3_bf16(dw[0], dw[1], scale), cvt4_e4m3_bf16(dw[2], dw[3], scale),
                                cvt4_e4m3_bf16(dw[4], dw[5], scale), cvt4_e4m3_bf16(dw[6], dw[7], scale));
    *reinterpret_cast<uint4 *>(ep.q + row * ep.I + dbase + 16 * h) = qv;
    if (h == 0) ep.s[row * (ep.I / 32) + dbase / 32] = (uint8_t)b;
  }
}

// One TM x 256 output tile (rows ti.row0 .. min(ti.row0 + TM, ti.row_end)).
// Row n of B_g starts at B + g * bexp + n * ldb (bytes; its scale bytes at
// Bs + (g * bexp + n * ldb) / 32): ldb = K, bexp = N K for B [G, N, K], and
// ldb = G K, bexp = K for the transposed column-wise copy of a stacked
// [G K, N] weight (the data-gradient operand).
// EPI: false = the plain store of the product, true = the fused gate_up
// epilogue (B rows permuted as swiglu_w_row describes; `out` unused).
template <bool OUT_F32, int TM, bool EPI = false>
__device__ __forceinline__ void mx3_tile(const uint8_t *__restrict__ A,
                                         const uint8_t *__restrict__ As,
                                         const uint8_t *__restrict__ B,
                                         const uint8_t *__restrict__ Bs, int64_t N, int64_t K,
                                         int64_t ldb, int64_t bexp, const TileInfo &ti,
                                         uint8_t *lds, void *__restrict__ out,
                                         const SwigluEpi *ep = nullptr) {
  using C = Mx3<TM>;
  constexpr int FI = C::FI, FJ = C::FJ, TN = C::TN;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1, h = lane >> 5, r32 = lane & 31;
  const uint32_t KS = (uint32_t)(K / 32), Ku = (uint32_t)K;
  const int rows_a = (int)min(ti.row_end - ti.row0, (int64_t)TM);
  const int rows_b = (int)min(N - ti.n0, (int64_t)TN);
  Mx3Src<TM> L;
  L.Ab = A + ti.row0 * K;
  L.Bb = B + ti.g * bexp + ti.n0 * ldb;
  L.dst = __builtin_amdgcn_readfirstlane(lds_addr(lds) + (uint32_t)wave * 1024u);
  // ring chunk c = 256 i + tid: row c / 4, physical chunk c % 4, which holds
  // logical chunk (c % 4) ^ ((row / 4) % 4)
#pragma unroll
  for (int i = 0; i < C::CA; ++i) {
    const int c = tid + 256 * i, r = c >> 2, k = (c & 3) ^ ((r >> 2) & 3);
    L.oa[i] = (uint32_t)min(r, rows_a - 1) * Ku + 16u * k;
  }
  if (EPI) L.Bb = B + ti.g * bexp;  // whole expert: rows picked by swiglu_w_row
#pragma unroll
  for (int i = 0; i < C::CB; ++i) {
    const int c = tid + 256 * i, r = c >> 2, k = (c & 3) ^ ((r >> 2) & 3);
    const int64_t wr = EPI ? swiglu_w_row(r, ti.n0 / TN, N / 2) : (int64_t)min(r, rows_b - 1);
    L.ob[i] = (uint32_t)wr * (uint32_t)ldb + 16u * k;
  }
  Mx3Lane o;
  {
    const int ra = wm * (TM / 2) + r32, rb = wn * 128 + r32;
    o.a_lo = mx3_off(ra, h);
    o.a_hi = mx3_off(ra, 2 + h);
    o.b_lo = TM * 64 + mx3_off(rb, h);
    o.b_hi = TM * 64 + mx3_off(rb, 2 + h);
    // group g = row / 16 starts at byte g * KS * 16; row rr of it at 4 rr
    o.sa = (ra >> 4) * (int)KS * 16 + (ra & 15) * 4;
    o.sb = ((TM + rb) >> 4) * (int)KS * 16 + ((TM + rb) & 15) * 4;
    o.ks = (int)KS;
  }
  // scale bytes of the tile's rows (A rows, then B rows) in groups of 16
  // rows, each group dword-major: dword dw of row 16 g + rr sits at dword
  // (g * KS/4 + dw) * 16 + rr.  A load instruction (64 consecutive dwords of
  // the area) reads 16 bytes from each of 16 rows; the 32 lanes reading one
  // block of 32 rows hit two runs of 16 consecutive dwords.
  {
    const uint8_t *Asb = As + ti.row0 * (int64_t)KS;
    const uint8_t *Bsb = Bs + (ti.g * bexp + ti.n0 * ldb) / 32;
    const int64_t ldbs = ldb / 32;
    const uint32_t sbase =
        __builtin_amdgcn_readfirstlane(lds_addr(lds) + C::NSLOT * C::SLOT + (uint32_t)wave * 256u);
    const int dpr = (int)(KS / 4);                  // dwords per row
    const int nq = (C::ROWS * dpr + 255) / 256;     // passes of 256 dwords
    for (int q = 0; q < nq; ++q) {
      const int d = 256 * q + tid;
      const int g = d / (16 * dpr), rem = d - g * 16 * dpr;
      const int row = min(16 * g + (rem & 15), C::ROWS - 1), dw = rem >> 4;
      const int64_t brow = EPI ? swiglu_w_row(row - TM, ti.n0 / TN, N / 2) - ti.n0
                               : (int64_t)min(row - TM, rows_b - 1);
      const uint8_t *src = row < TM ? Asb + (int64_t)min(row, rows_a - 1) * KS + 4 * dw
                                    : Bsb + brow * ldbs + 4 * dw;
      dma4(src, sbase + 1024u * (uint32_t)q);
    }
  }

  v16f acc[FI][FJ];
#pragma unroll
  for (int i = 0; i < FI; ++i)
#pragma unroll
    for (int j = 0; j < FJ; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  const int nk = (int)(K / 64);  // even, >= 2
  mx3_issue<TM>(L, 0, 0);
  mx3_issue<TM>(L, 1, 1);
  mx3_issue<TM>(L, min(2, nk - 1), 2);
  vm_wait<2 * C::OPS>();  // the scale area and step 0
  __builtin_amdgcn_s_barrier();
  Mx3Frags<TM> F0, F1;
  mx3_read<TM>(lds, 0, 0, o, F0);
  int slot = 0;
  for (int kt = 0; kt < nk; kt += 2) {
    mx3_step<TM>(L, lds, o, kt, nk, slot, acc, F0, F1);
    slot = slot == 2 ? 0 : slot + 1;
    mx3_step<TM>(L, lds, o, kt + 1, nk, slot, acc, F1, F0);
    slot = slot == 2 ? 0 : slot + 1;
  }
  vm_wait<0>();  // no load may still target this workgroup's LDS at exit
  if (EPI) {
#pragma unroll
    for (int i = 0; i < FI; ++i)
#pragma unroll
      for (int jj = 0; jj < FJ / 2; ++jj)
        swiglu_store(acc[i][2 * jj], acc[i][2 * jj + 1], *ep, ti.row0, ti.row_end,
                     wm * (TM / 2) + 32 * i, ti.n0 / 2 + 64 * wn + 32 * jj);
  } else {
#pragma unroll
    for (int i = 0; i < FI; ++i)
#pragma unroll
      for (int j = 0; j < FJ; ++j)
        mx3_store<OUT_F32>(acc[i][j], out, N, ti.row0, ti.row_end, ti.n0,
                           wm * (TM / 2) + 32 * i, wn * 128 + 32 * j);
  }
}

__device__ __forceinline__ v8i mw_frag(const uint8_t *p_lo, const uint8_t *p_hi) {
  const uint4 lo = *reinterpret_cast<const uint4 *>(p_lo);
  const uint4 hi = *reinterpret_cast<const uint4 *>(p_hi);
  return v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
}

// ------------------------------- MXFP8, eight waves, 128-byte ring steps
// The 256 x 256 tile with 8 waves (two per SIMD, each 128 x 64 outputs) and
// a ring of two slots, each holding one 128-K step: 128 bytes of every tile
// row (A rows, then B rows) plus one 4-byte word per row with the row's four
// E8M0 scale bytes of the step.  A load instruction then reads whole
// 128-byte lines (8 lanes per row, 64 rows per instruction): measured, a CU
// streams ~107 GB/s that way against ~64 GB/s when each row contributes half
// a line per step, and the tile needs ~64 GB/s at the matrix core's rate.
// The scales travel with the data, so nothing is preloaded and any
// K % 128 == 0 fits.  Rows are 8 chunks of 16 bytes, chunk c of row r stored
// at c ^ (r % 8).
// Schedule of step k (slot s = k % 2): the first half (64 K) multiplies the
// fragments read before it and reads the second half's fragments of slot s;
// then every wave waits for its loads of step k+1 (slot s ^ 1) and for its
// LDS reads, and meets the others at the barrier (step k+1 published, slot
// s no longer read); the second half multiplies, requests step k+2 into
// slot s and reads step k+1's first-half fragments.  So a step's loads have
// one full step to arrive.  A lane holds one set of fragments, each
// replaced right after its last use.
template <int TM>
struct Mq {
  static constexpr int TN = 256, ROWS = TM + TN;
  static constexpr int DATA = ROWS * 128;     // operand bytes of a slot
  static constexpr int SLOT = DATA + 2048;    // + scale words (512 entries)
  static constexpr int NSLOT = 2, LDS = NSLOT * SLOT;
  static constexpr int CA = TM / 64, CB = TN / 64;  // 16-byte loads per lane per step
  static constexpr int OPS = CA + CB + 1;           // + one scale word per lane
  static constexpr int FI = TM / 64, FJ = 2;
};

// 16 bytes per lane from global `sbase + voff` (sbase wave-uniform, in
// scalar registers) into LDS at m0 + 16 * lane.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16s(const void *sbase, uint32_t voff, uint32_t m0) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sbase),
               "s"(m0)
               : "memory", "m0");
}
#pragma clang diagnostic pop

__device__ __forceinline__ const uint8_t *uniform_ptr(const uint8_t *p) {
  const uint64_t u = (uint64_t)(uintptr_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)u);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(u >> 32));
  return reinterpret_cast<const uint8_t *>((uintptr_t)(((uint64_t)hi << 32) | lo));
}

template <int TM>
struct MqSrc {
  const uint8_t *Ab, *Bb;                   // operand panels (wave-uniform)
  const uint8_t *sp;                        // this lane's scale-word row (k = 0)
  uint32_t oa[Mq<TM>::CA], ob[Mq<TM>::CB];  // per-lane chunk sources at k = 0
  uint32_t dst;                             // LDS address of slot 0, this wave's lanes
  uint32_t sdst;                            // LDS address of slot 0's scale words, this wave
};

template <int TM>
__device__ __forceinline__ void mq_load(const MqSrc<TM> &L, int q, uint32_t kb, int slot) {
  using C = Mq<TM>;
  const uint32_t sl = (uint32_t)slot * C::SLOT;
  if (q < C::CA)
    dma16s(L.Ab, L.oa[q] + kb, L.dst + sl + q * 8192);
  else if (q < C::CA + C::CB)
    dma16s(L.Bb, L.ob[q - C::CA] + kb, L.dst + sl + TM * 128 + (q - C::CA) * 8192);
  else
    dma4(L.sp + kb / 32, L.sdst + sl);
}

template <int TM>
struct MqFrags {
  v8i a[Mq<TM>::FI], b[Mq<TM>::FJ];
  int sa[Mq<TM>::FI], sb[Mq<TM>::FJ];
};

// The ring's 16-byte chunk swizzle: logical chunk c of LDS row r sits at
// physical chunk c ^ mq_swz(r).  A fragment read (16 bytes per lane) serves
// 16 lanes, i.e. 16 consecutive rows, per LDS cycle, and two 128-byte rows
// share one 256-byte row of banks, so the key is taken from r / 2: the 16
// rows of a read then reach 16 distinct bank groups (r % 8 as the key left
// rows r and r + 8 on the same banks, a 2-way conflict on every read).
__device__ __forceinline__ int mq_swz(int r) { return (r >> 1) & 7; }

// Per-lane LDS offsets: first A / B row's chunks h and 2 + h of K-half 0
// (K-half t adds 64 bytes before the swizzle: chunk 4 t + x), fragments 32
// rows (4096 bytes) apart; scale bytes of the first A / B row, block h.
struct MqLane {
  int a0, a1, b0, b1;  // chunk byte offsets for half 0
  int x;               // mq_swz(row) (the same for every fragment row of the lane)
  int sa, sb;          // scale byte offsets (half 0)
};

template <int TM>
__device__ __forceinline__ void mq_read_one(const uint8_t *lds, int slot, int half,
                                            const MqLane &o, int f, MqFrags<TM> &F) {
  using C = Mq<TM>;
  const uint8_t *cur = lds + slot * C::SLOT;
  // chunk (4 half + h) ^ x = chunk (h ^ x) with bit 2 flipped by half
  const int hx = half * 64;
  if (f < C::FI) {
    F.a[f] = mw_frag(cur + (o.a0 ^ hx) + 4096 * f, cur + (o.a1 ^ hx) + 4096 * f);
    F.sa[f] = cur[C::DATA + o.sa + 2 * half + 128 * f];
  } else {
    const int g = f - C::FI;
    F.b[g] = mw_frag(cur + (o.b0 ^ hx) + 4096 * g, cur + (o.b1 ^ hx) + 4096 * g);
    F.sb[g] = cur[C::DATA + o.sb + 2 * half + 128 * g];
  }
}

// One K-half: FI x FJ MFMAs on F, in the order (b0, a0..), (b1, a0..); each
// fragment is replaced by fragment f of (rslot, rhalf) after its last use;
// load q of `lq` goes out after MFMA q when lq.k >= 0.
template <int TM>
__device__ __forceinline__ void mq_half(const MqSrc<TM> &L, const uint8_t *lds, const MqLane &o,
                                        v16f (&acc)[Mq<TM>::FI][Mq<TM>::FJ], MqFrags<TM> &F,
                                        int rslot, int rhalf, bool loads, uint32_t kb, int lslot,
                                        bool MF = true) {
  using C = Mq<TM>;
  constexpr int FI = C::FI;
#pragma unroll
  for (int m = 0; m < 2 * FI; ++m) {
    const int j = m / FI, i = m % FI;
    if (MF)
      acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(F.b[j], F.a[i], acc[i][j], 0,
                                                                   0, 0, F.sb[j], 0, F.sa[i]);
    if (loads) {
      // OPS loads spread over the 2 FI MFMAs (two per MFMA while needed)
      constexpr int PER = (C::OPS + 2 * FI - 1) / (2 * FI);
#pragma unroll
      for (int q = PER * m; q < PER * m + PER && q < C::OPS; ++q) mq_load<TM>(L, q, kb, lslot);
    }
    if (m == FI - 1) mq_read_one<TM>(lds, rslot, rhalf, o, FI, F);          // b0
    if (m >= FI) mq_read_one<TM>(lds, rslot, rhalf, o, i, F);              // a_i
    if (m == 2 * FI - 1) mq_read_one<TM>(lds, rslot, rhalf, o, FI + 1, F);  // b1
    __builtin_amdgcn_sched_barrier(0);
  }
}

// bf16 epilogue through LDS: each wave writes its rounded accumulators into a
// TM x 256 bf16 tile (row pitch 512 bytes, 16-byte chunk x of row r at
// x ^ (r % 32)), then every lane stores 16 bytes of a row, so one store
// instruction writes two whole 512-byte rows (four full 128-byte lines
// each) instead of 32 bytes of 32 rows.
template <int TM>
__device__ __forceinline__ void mq_store_staged(const v16f (&acc)[Mq<TM>::FI][Mq<TM>::FJ],
                                                uint8_t *lds, const TileInfo &ti, int64_t N,
                                                void *__restrict__ out,
                                                const float *bias = nullptr) {
  static_assert(TM * 512 <= Mq<TM>::LDS, "staged tile fits the ring");
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 2, wn = wave & 3, h = lane >> 5, r32 = lane & 31;
#pragma unroll
  for (int i = 0; i < Mq<TM>::FI; ++i) {
    const int R = wm * (TM / 2) + 32 * i + r32;
#pragma unroll
    for (int j = 0; j < Mq<TM>::FJ; ++j)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        // columns 64 wn + 32 j + 8 g + 4 h + 0..3: chunk 8 wn + 4 j + g, bytes 8 h ..
        const int x = 8 * wn + 4 * j + g;
        float f[4] = {acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2],
                      acc[i][j][4 * g + 3]};
        if (bias) {
          const int64_t col = ti.n0 + 64 * wn + 32 * j + 8 * g + 4 * h;
#pragma unroll
          for (int e = 0; e < 4; ++e) f[e] += bias[min(col + e, N - 1)];
        }
        const uint2 v = make_uint2(pk_bf16_rne(f[0], f[1]), pk_bf16_rne(f[2], f[3]));
        *reinterpret_cast<uint2 *>(lds + R * 512 + ((x ^ (R & 31)) * 16) + 8 * h) = v;
      }
  }
  __syncthreads();
  const int rows = (int)min(ti.row_end - ti.row0, (int64_t)TM);
  const int x = tid & 31;
  const int64_t col = ti.n0 + 8 * x;
  const bool vec = (N & 7) == 0 && col + 7 < N;
#pragma unroll 4
  for (int it = 0; it < TM / 16; ++it) {
    const int R = 16 * it + (tid >> 5);
    const uint4 v = *reinterpret_cast<const uint4 *>(lds + R * 512 + ((x ^ (R & 31)) * 16));
    if (R >= rows) continue;
    uint16_t *orow = static_cast<uint16_t *>(out) + (ti.row0 + R) * N;
    if (vec) {
      *reinterpret_cast<uint4 *>(orow + col) = v;
    } else {
      const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (col + e < N) orow[col + e] = (uint16_t)(w[e >> 1] >> (16 * (e & 1)));
    }
  }
}

template <bool OUT_F32, int TM>
__device__ __forceinline__ void mq_tile(const uint8_t *__restrict__ A,
                                        const uint8_t *__restrict__ As,
                                        const uint8_t *__restrict__ B,
                                        const uint8_t *__restrict__ Bs, int64_t N, int64_t K,
                                        int64_t ldb, int64_t bexp, const TileInfo &ti,
                                        uint8_t *lds, void *__restrict__ out,
                                        const float *bias) {
  using C = Mq<TM>;
  constexpr int FI = C::FI, FJ = C::FJ, TN = C::TN;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 2, wn = wave & 3, h = lane >> 5, r32 = lane & 31;
  const int64_t KS = K / 32;
  const uint32_t Ku = (uint32_t)K;
  const int rows_a = (int)min(ti.row_end - ti.row0, (int64_t)TM);
  const int rows_b = (int)min(N - ti.n0, (int64_t)TN);
  MqSrc<TM> L;
  L.Ab = uniform_ptr(A + ti.row0 * K);
  L.Bb = uniform_ptr(B + ti.g * bexp + ti.n0 * ldb);
  L.dst = __builtin_amdgcn_readfirstlane(lds_addr(lds) + (uint32_t)wave * 1024u);
  L.sdst = __builtin_amdgcn_readfirstlane(lds_addr(lds) + C::DATA + (uint32_t)wave * 256u);
  // load q, lane tid: row 64 q + tid / 8 of the operand, physical chunk
  // tid % 8 holding logical chunk (tid % 8) ^ mq_swz(row); rows past the
  // expert's end or past N load a clamped valid row
#pragma unroll
  for (int q = 0; q < C::CA; ++q) {
    const int r = 64 * q + (tid >> 3), c = (tid & 7) ^ mq_swz(r);
    L.oa[q] = (uint32_t)min(r, rows_a - 1) * Ku + 16u * c;
  }
#pragma unroll
  for (int q = 0; q < C::CB; ++q) {
    const int r = 64 * q + (tid >> 3), c = (tid & 7) ^ mq_swz(r);
    L.ob[q] = (uint32_t)min(r, rows_b - 1) * (uint32_t)ldb + 16u * c;
  }
  // scale word of lane tid: tile row tid (A rows first; lanes past the
  // tile's rows fetch a valid row into the unused entries)
  {
    const int r = min(tid, C::ROWS - 1);
    L.sp = r < TM ? As + (ti.row0 + min(r, rows_a - 1)) * KS
                  : Bs + (ti.g * bexp + ti.n0 * ldb) / 32 + (int64_t)min(r - TM, rows_b - 1) * (ldb / 32);
  }
  MqLane o;
  {
    const int ra = wm * (TM / 2) + r32, rb = wn * 64 + r32;
    o.x = mq_swz(r32);
    o.a0 = ra * 128 + ((h ^ o.x) * 16);
    o.a1 = ra * 128 + (((2 + h) ^ o.x) * 16);
    o.b0 = TM * 128 + rb * 128 + ((h ^ o.x) * 16);
    o.b1 = TM * 128 + rb * 128 + (((2 + h) ^ o.x) * 16);
    o.sa = ra * 4 + h;
    o.sb = (TM + rb) * 4 + h;
  }

  v16f acc[FI][FJ];
#pragma unroll
  for (int i = 0; i < FI; ++i)
#pragma unroll
    for (int j = 0; j < FJ; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  const int nk = (int)(K / 128);  // >= 1
#pragma unroll
  for (int q = 0; q < C::OPS; ++q) mq_load<TM>(L, q, 0u, 0);
#pragma unroll
  for (int q = 0; q < C::OPS; ++q) mq_load<TM>(L, q, (uint32_t)min(1, nk - 1) * 128u, 1);
  vm_wait<C::OPS>();  // step 0
  __builtin_amdgcn_s_barrier();
  MqFrags<TM> F;
#pragma unroll
  for (int f = 0; f < FI + FJ; ++f) mq_read_one<TM>(lds, 0, 0, o, f, F);
  for (int kt = 0; kt < nk; ++kt) {
    const int slot = kt & 1;
    mq_half<TM>(L, lds, o, acc, F, slot, 1, false, 0u, 0);
    vm_wait<0>();  // own loads of step kt+1 arrived
    lgkm_wait0();  // own reads of this slot done
    __builtin_amdgcn_s_barrier();
    // past the last step: requests repeat it and reads take step nk-1's
    // first half again (in bounds, never used)
    const uint32_t kb = (uint32_t)min(kt + 2, nk - 1) * 128u;
    mq_half<TM>(L, lds, o, acc, F, kt + 1 < nk ? slot ^ 1 : slot, 0, true, kb, slot);
  }
  vm_wait<0>();  // no load may still target this workgroup's LDS at exit
  if (OUT_F32) {
#pragma unroll
    for (int i = 0; i < FI; ++i)
#pragma unroll
      for (int j = 0; j < FJ; ++j)
        mx3_store<OUT_F32>(acc[i][j], out, N, ti.row0, ti.row_end, ti.n0,
                           wm * (TM / 2) + 32 * i, wn * 64 + 32 * j, bias);
  } else {
    lgkm_wait0();
    __builtin_amdgcn_s_barrier();  // the ring is no longer read: stage the tile there
    mq_store_staged<TM>(acc, lds, ti, N, out, bias);
  }
}

template <bool OUT_F32, bool BIAS>
__global__ __launch_bounds__(512, 1) void k_gemm_mxfp8_q(
    const uint8_t *__restrict__ A, const uint8_t *__restrict__ As,
    const uint8_t *__restrict__ B, const uint8_t *__restrict__ Bs,
    const int64_t *__restrict__ offsets, int64_t G, int64_t N, int64_t K, int64_t ntn,
    int64_t ldb, int64_t bexp, void *__restrict__ out, const float *__restrict__ bias) {
  static_assert(Mq<128>::LDS <= Mq<256>::LDS, "LDS of the half tile");
  __shared__ __attribute__((aligned(16))) uint8_t lds[Mq<256>::LDS];
  __shared__ int64_t sh[4];
  TileInfo ti;
  if (!lookup_row_tile<256, 256>(offsets, G, ntn, ti, sh)) return;
  const float *bg = BIAS ? bias + ti.g * N : nullptr;
  if (ti.row_end - ti.row0 <= 128)
    mq_tile<OUT_F32, 128>(A, As, B, Bs, N, K, ldb, bexp, ti, lds, out, bg);
  else
    mq_tile<OUT_F32, 256>(A, As, B, Bs, N, K, ldb, bexp, ti, lds, out, bg);
}

// ------------------------------------------ MXFP8, persistent eight waves
// k_gemm_mxfp8_q as a persistent kernel: one workgroup per CU walks its
// tiles (those of its XCD's contiguous range, 32 apart) with one unbroken
// stream of ring steps, so the first two steps of tile n+1 are loaded while
// tile n finishes and no tile starts with an empty ring.  Tile n's output
// leaves by buffer stores issued right after its last step (rows past the
// tile's end get an offset beyond the buffer, which the hardware drops); the
// first step of tile n+1 waits for them with its own loads, which were
// issued before them (only loads keep their order in vmcnt, so a wait that
// let the stores stay in flight could release early).  On an
// expert's last tile of at most 128 rows the four waves of rows 128..255
// skip their MFMAs (their rows are beyond the tile).  The tile list is made
// once at the start: a scan of the per-expert tile counts (in the ring's
// LDS, before any ring load), then each tile found by binary search.
constexpr int QP_MAXT = 256;  // tiles per workgroup
// Store offset of a lane with nothing to store: past the output (which is
// smaller than 2^31 bytes) without wrapping, so the hardware range check
// drops it.
constexpr uint32_t QP_OOB = 0x80000000u;

struct QpTile {
  int32_t row0, row_end, g, n0;
};

// Exclusive prefix of v over the 512 threads (thread order) plus `carry`,
// which then grows by the 512 values' sum.  wsum: 8 shared slots.
__device__ __forceinline__ int32_t qp_scan512(int32_t v, int32_t &carry, int32_t *wsum) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int32_t incl = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int32_t t = __shfl_up(incl, o, 64);
    if (lane >= o) incl += t;
  }
  if (lane == 63) wsum[wave] = incl;
  __syncthreads();
  int32_t before = carry, all = 0;
#pragma unroll
  for (int w = 0; w < 8; ++w) {
    before += w < wave ? wsum[w] : 0;
    all += wsum[w];
  }
  carry += all;
  __syncthreads();
  return before + incl - v;
}

// 4 x 4 transpose of 4-dword groups inside every quad of lanes (lanes
// 4a + b, b = 0..3): group k of lane b ends up holding what group b of lane
// k held, in two exchange stages with the lanes b ^ 1 and b ^ 2 (DPP quad
// permutes, selects only, so the groups stay in registers).  Used to turn a
// 32 x 32 accumulator layout (one row per lane) into stores that each write
// eight whole 128-byte rows.
typedef uint32_t pqm_v16u __attribute__((ext_vector_type(16)));
template <int S>
__device__ __forceinline__ pqm_v16u quad_stage(pqm_v16u v, bool hi) {
  pqm_v16u r = v;
  constexpr int ctrl = S == 1 ? 0xB1 : 0x4E;  // quad_perm lane b ^ S
#pragma unroll
  for (int q = 0; q < 8; ++q) {  // the 8 registers of the groups g0 with bit S clear
    const int g0 = S == 1 ? 2 * (q >> 2) : (q >> 2), e = q & 3;
    const int x0 = 4 * g0 + e, x1 = 4 * (g0 | S) + e;
    // the partner's registers (each select takes its moved operand directly)
    const uint32_t p1 = (uint32_t)__builtin_amdgcn_mov_dpp((int)v[x1], ctrl, 0xF, 0xF, false);
    const uint32_t p0 = (uint32_t)__builtin_amdgcn_mov_dpp((int)v[x0], ctrl, 0xF, 0xF, false);
    r[x0] = !hi ? v[x0] : p1;
    r[x1] = hi ? v[x1] : p0;
  }
  return r;
}
__device__ __forceinline__ pqm_v16u quad_transpose(pqm_v16u v, int b) {
  return quad_stage<2>(quad_stage<1>(v, (b & 1) != 0), (b & 2) != 0);
}

// bias: the expert's bias row (binary32, N columns) added before the output
// rounding, or null.
template <bool OUT_F32>
__device__ __forceinline__ void qp_store(const v16f (&acc)[4][2], __amdgpu_buffer_rsrc_t rs,
                                         const QpTile &t, int64_t N, const float *bias = nullptr) {
  typedef unsigned int u32x4 __attribute__((__vector_size__(16)));
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 2, wn = wave & 3, h = lane >> 5, r32 = lane & 31;
  const uint32_t Nu = (uint32_t)N;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const v16f &a = acc[i][j];
      const int cb = t.n0 + wn * 64 + 32 * j;
      if (OUT_F32) {
        // binary32: group g of lane (h, r) is row r at columns 8 g + 4 h ..
        // + 3; after the quad transpose group k of lane (h, 4 a + b) is row
        // 4 a + k at columns 4 (2 b + h) .. + 3, so each store writes eight
        // whole 128-byte rows
        const int b = r32 & 3, a4 = r32 >> 2;
        const pqm_v16u v = quad_transpose(__builtin_bit_cast(pqm_v16u, a), b);
        const uint32_t col = (uint32_t)(cb + 4 * (2 * b + h));
        float bb[4] = {0.0f, 0.0f, 0.0f, 0.0f};
        if (bias) {
#pragma unroll
          for (int e = 0; e < 4; ++e) bb[e] = bias[min(col + e, Nu - 1u)];
        }
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const int rowk = t.row0 + wm * 128 + 32 * i + 4 * a4 + k;
          const uint32_t off =
              rowk < t.row_end && col < Nu ? ((uint32_t)rowk * Nu + col) * 4u : QP_OOB;
          u32x4 w = {v[4 * k], v[4 * k + 1], v[4 * k + 2], v[4 * k + 3]};
          if (bias) {
#pragma unroll
            for (int e = 0; e < 4; ++e) w[e] = __float_as_uint(__uint_as_float(w[e]) + bb[e]);
          }
          __builtin_amdgcn_raw_buffer_store_b128(w, rs, (int)off, 0, 0);
        }
      }
    }
    if (!OUT_F32) {
      // bf16: lane (h, r) holds row r's columns 16 p + 4 h .. + 3 (x) and
      // 16 p + 8 + 4 h .. + 3 (y) of the fragment's 32; packed in pairs, one
      // lane swap of the upper half-wave's x with the lower half-wave's y
      // leaves lane (0, r) with chunk 2 p (its own x, then lane (1, r)'s) and
      // lane (1, r) with chunk 2 p + 1 (lane (0, r)'s y, then its own): chunk
      // 4 j + 2 p + h of the wave's 64 columns.  A quad transpose of those 4
      // chunks leaves in chunk k of lane (h, 4 a + b) row 4 a + k's chunk
      // 2 b + h, so each store writes eight whole 128-byte rows
      pqm_v16u v;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
#pragma unroll
        for (int p = 0; p < 2; ++p) {
          const v16f &a = acc[i][j];
          float x[4], y[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            x[e] = a[8 * p + e];
            y[e] = a[8 * p + 4 + e];
          }
          if (bias) {
            // runs of 4 columns start on a multiple of 4 and N % 8 == 0, so a
            // run is inside N or wholly past it (then any run will do)
            const uint32_t c = (uint32_t)(t.n0 + wn * 64 + 32 * j + 16 * p + 4 * h);
            const float *bx = bias + min(c, Nu - 4u), *by = bias + min(c + 8, Nu - 4u);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              x[e] += bx[e];
              y[e] += by[e];
            }
          }
          const auto s0 = __builtin_amdgcn_permlane32_swap(pk_bf16_rne(x[0], x[1]),
                                                           pk_bf16_rne(y[0], y[1]), false, false);
          const auto s1 = __builtin_amdgcn_permlane32_swap(pk_bf16_rne(x[2], x[3]),
                                                           pk_bf16_rne(y[2], y[3]), false, false);
          const int m = 2 * j + p;
          v[4 * m] = s0[0];
          v[4 * m + 1] = s1[0];
          v[4 * m + 2] = s0[1];
          v[4 * m + 3] = s1[1];
        }
      }
      const int b = r32 & 3, a4 = r32 >> 2;
      v = quad_transpose(v, b);
      const uint32_t col = (uint32_t)(t.n0 + wn * 64 + 8 * (2 * b + h));
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int rowk = t.row0 + wm * 128 + 32 * i + 4 * a4 + k;
        const uint32_t off =
            rowk < t.row_end && col < Nu ? ((uint32_t)rowk * Nu + col) * 2u : QP_OOB;
        const u32x4 w = {v[4 * k], v[4 * k + 1], v[4 * k + 2], v[4 * k + 3]};
        __builtin_amdgcn_raw_buffer_store_b128(w, rs, (int)off, 0, 0);
      }
    }
  }
}

// Fused gate_up epilogue on the eight-wave layout: wave (wm, wn) of tile tn
// holds, per row, gate values in its fragment j = 0 and up values in j = 1
// for the 32 D columns 128 tn + 32 wn + 0..31 (one MXFP8 block): the
// transposed accumulator gives lane h * 32 + r the fragment columns
// 8 g + 4 h + e (g, e = 0..3) as registers 4 g + e, and tile column
// c = 64 wn + 32 j + 8 g + 4 h + e is made gate (j = 0) or up (j = 1) of
// D column dcol = 128 tn + 32 wn + 16 h + 4 g + e, i.e. W row dcol or
// I + dcol.  A lane then holds 16 consecutive D columns.
__device__ __forceinline__ int64_t qp_swiglu_w_row(int c, int64_t tn, int64_t I) {
  const int wn = c >> 6, j = (c >> 5) & 1, g = (c >> 3) & 3, hh = (c >> 2) & 1, e = c & 3;
  const int64_t dcol = 128 * tn + 32 * wn + 16 * hh + 4 * g + e;
  return j ? I + dcol : dcol;
}

// Loader of one 256 x 256 tile (as in mq_tile); EPI: B rows permuted as
// qp_swiglu_w_row describes (N = 2 I, whole tiles).
template <bool EPI = false>
__device__ __forceinline__ void qp_loader(MqSrc<256> &L, const QpTile &t,
                                          const uint8_t *__restrict__ A,
                                          const uint8_t *__restrict__ As,
                                          const uint8_t *__restrict__ B,
                                          const uint8_t *__restrict__ Bs, int64_t N, int64_t K,
                                          int64_t ldb, int64_t bexp) {
  using C = Mq<256>;
  const int tid = threadIdx.x;
  const int64_t KS = K / 32;
  const uint32_t Ku = (uint32_t)K;
  const int rows_a = min(t.row_end - t.row0, 256);
  const int rows_b = (int)min(N - t.n0, (int64_t)256);
  const int64_t tn = t.n0 / 256;
  L.Ab = uniform_ptr(A + (int64_t)t.row0 * K);
  L.Bb = uniform_ptr(B + t.g * bexp + (EPI ? 0 : t.n0 * ldb));
#pragma unroll
  for (int q = 0; q < C::CA; ++q) {
    const int r = 64 * q + (tid >> 3), c = (tid & 7) ^ mq_swz(r);
    L.oa[q] = (uint32_t)min(r, rows_a - 1) * Ku + 16u * c;
  }
#pragma unroll
  for (int q = 0; q < C::CB; ++q) {
    const int r = 64 * q + (tid >> 3), c = (tid & 7) ^ mq_swz(r);
    const int64_t wr = EPI ? qp_swiglu_w_row(r, tn, N / 2) : (int64_t)min(r, rows_b - 1);
    L.ob[q] = (uint32_t)wr * (uint32_t)ldb + 16u * c;
  }
  const int r = tid;  // 512 lanes, 512 tile rows
  const int64_t wr = EPI ? qp_swiglu_w_row(max(r - 256, 0), tn, N / 2) - t.n0
                         : (int64_t)min(r - 256, rows_b - 1);
  L.sp = r < 256 ? As + ((int64_t)t.row0 + min(r, rows_a - 1)) * KS
                 : Bs + (t.g * bexp + t.n0 * ldb) / 32 + wr * (ldb / 32);
}

// The fused epilogue of one tile: D = bf16(silu(bf16 gate) bf16 up p) as
// pqm_swiglu_prob computes it, then its row-wise MXFP8 block (this lane's
// 16 columns and the other half's 16), stored with buffer stores whose
// count is the same in every wave: 4 of 16 bytes (q) and 4 of one byte (s)
// per lane, lanes without a value getting a dropped offset.
__device__ __forceinline__ void qp_swiglu_store(const v16f (&acc)[4][2], const float (&pr)[4],
                                                __amdgpu_buffer_rsrc_t rq,
                                                __amdgpu_buffer_rsrc_t rs, const QpTile &t,
                                                int64_t I) {
  typedef unsigned int u32x4 __attribute__((__vector_size__(16)));
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 2, wn = wave & 3, h = lane >> 5, r32 = lane & 31;
  const uint32_t dbase = (uint32_t)(t.n0 / 2 + 32 * wn), Iu = (uint32_t)I;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = t.row0 + wm * 128 + 32 * i + r32;
    const bool ok = row < t.row_end;
    uint32_t dw[8];  // D columns dbase + 16 h + 2 k, + 1
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int g = k >> 1, e = 2 * (k & 1);
      const uint32_t gw = pk_bf16_rne(acc[i][0][4 * g + e], acc[i][0][4 * g + e + 1]);
      const uint32_t uw = pk_bf16_rne(acc[i][1][4 * g + e], acc[i][1][4 * g + e + 1]);
      dw[k] = pk_bf16_rne(swiglu_f32(bf16_lo_f32(gw), bf16_lo_f32(uw), pr[i]),
                          swiglu_f32(bf16_hi_f32(gw), bf16_hi_f32(uw), pr[i]));
    }
    uint32_t mm = 0;
#pragma unroll
    for (int k = 0; k < 8; ++k) mm = pk_max_u16(mm, dw[k] & 0x7FFF7FFFu);
    mm = max(mm & 0xFFFFu, mm >> 16);
    {
      const auto sw = __builtin_amdgcn_permlane32_swap(mm, mm, false, false);
      mm = max(sw[0], sw[1]);
    }
    const uint32_t b = mx_scale_byte(mm);
    const float scale = __uint_as_float(b << 23);
    const u32x4 qv = {cvt4_e4m3_bf16(dw[0], dw[1], scale), cvt4_e4m3_bf16(dw[2], dw[3], scale),
                      cvt4_e4m3_bf16(dw[4], dw[5], scale), cvt4_e4m3_bf16(dw[6], dw[7], scale)};
    const uint32_t qoff = ok ? (uint32_t)row * Iu + dbase + 16u * (uint32_t)h : QP_OOB;
    const uint32_t soff = ok && h == 0 ? (uint32_t)row * (Iu / 32) + dbase / 32 : QP_OOB;
    __builtin_amdgcn_raw_buffer_store_b128(qv, rq, (int)qoff, 0, 0);
    __builtin_amdgcn_raw_buffer_store_b8((uint8_t)b, rs, (int)soff, 0, 0);
  }
}

template <bool OUT_F32, bool EPI>
__device__ __forceinline__ void k_gemm_mxfp8_qp_body(
    const uint8_t *__restrict__ A, const uint8_t *__restrict__ As,
    const uint8_t *__restrict__ B, const uint8_t *__restrict__ Bs,
    const int64_t *__restrict__ offsets, int64_t G, int64_t N, int64_t K, int64_t ntn,
    int64_t ldb, int64_t bexp, void *__restrict__ out, uint32_t out_bytes, const SwigluEpi &ep,
    const float *__restrict__ bias);

template <bool OUT_F32, bool BIAS>
__global__ __launch_bounds__(512, 1) void k_gemm_mxfp8_qp(
    const uint8_t *__restrict__ A, const uint8_t *__restrict__ As,
    const uint8_t *__restrict__ B, const uint8_t *__restrict__ Bs,
    const int64_t *__restrict__ offsets, int64_t G, int64_t N, int64_t K, int64_t ntn,
    int64_t ldb, int64_t bexp, void *__restrict__ out, uint32_t out_bytes,
    const float *__restrict__ bias) {
  k_gemm_mxfp8_qp_body<OUT_F32, false>(A, As, B, Bs, offsets, G, N, K, ntn, ldb, bexp, out,
                                       out_bytes, SwigluEpi{nullptr, nullptr, 0, nullptr, nullptr},
                                       BIAS ? bias : nullptr);
}

template <bool OUT_F32, bool EPI>
__device__ __forceinline__ void k_gemm_mxfp8_qp_body(
    const uint8_t *__restrict__ A, const uint8_t *__restrict__ As,
    const uint8_t *__restrict__ B, const uint8_t *__restrict__ Bs,
    const int64_t *__restrict__ offsets, int64_t G, int64_t N, int64_t K, int64_t ntn,
    int64_t ldb, int64_t bexp, void *__restrict__ out, uint32_t out_bytes, const SwigluEpi &ep,
    const float *__restrict__ bias) {
  using C = Mq<256>;
  __shared__ __attribute__((aligned(16))) uint8_t lds[C::LDS];
  __shared__ QpTile tl[QP_MAXT];
  __shared__ int32_t wsum[8], nt_sh;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 2, wn = wave & 3, h = lane >> 5, r32 = lane & 31;

  // ---- tile list: per-expert counts of 256-row tiles, scanned into tpre
  int32_t *tpre = reinterpret_cast<int32_t *>(lds);  // G + 1 entries (checked on the host)
  {
    int32_t carry = 0;
    for (int64_t b0 = 0; b0 < G; b0 += 512) {
      const int64_t g = b0 + tid;
      const int32_t v = g < G ? (int32_t)((offsets[g + 1] - offsets[g] + 255) / 256) : 0;
      const int32_t x = qp_scan512(v, carry, wsum);
      if (g < G) tpre[g] = x;
    }
    if (tid == 0) tpre[G] = carry;
  }
  __syncthreads();
  {
    const int64_t real = (int64_t)tpre[G] * ntn;
    const int64_t per_xcd = (real + 7) / 8, nw = gridDim.x / 8;
    const int64_t lo = (blockIdx.x % 8) * per_xcd + blockIdx.x / 8;
    const int64_t hi = min((blockIdx.x % 8 + 1) * per_xcd, real);
    const int nt = lo < hi ? (int)((hi - lo + nw - 1) / nw) : 0;
    if (tid == 0) nt_sh = min(nt, QP_MAXT);
    for (int k = tid; k < nt && k < QP_MAXT; k += 512) {
      const int64_t T = lo + (int64_t)k * nw;
      const int32_t mt = (int32_t)(T / ntn);
      int a = 0, b = (int)G;  // largest g with tpre[g] <= mt (tpre[G] > mt)
      while (b - a > 1) {
        const int m = (a + b) >> 1;
        if (tpre[m] <= mt) a = m; else b = m;
      }
      QpTile t;
      t.g = a;
      t.row0 = (int32_t)(offsets[a] + (int64_t)(mt - tpre[a]) * 256);
      t.row_end = (int32_t)offsets[a + 1];
      t.n0 = (int32_t)((T % ntn) * 256);
      tl[k] = t;
    }
  }
  __syncthreads();  // the tile list is complete and tpre is no longer read
  const int nt = nt_sh;
  if (nt == 0) return;
  const int nk = (int)(K / 128);
  const int S = nt * nk;
  // EPI: out_bytes = M I (q); the scale array is M I / 32 bytes
  __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(EPI ? (void *)ep.q : out, (short)0,
                                                                (int)out_bytes, 0x00020000);
  __amdgpu_buffer_rsrc_t rss =
      __builtin_amdgcn_make_buffer_rsrc(ep.s, (short)0, (int)(out_bytes / 32), 0x00020000);
  float pr[4] = {0.0f, 0.0f, 0.0f, 0.0f};  // EPI: router probability of the lane's rows
  int32_t pidx[4] = {0, 0, 0, 0};

  MqSrc<256> L;
  L.dst = __builtin_amdgcn_readfirstlane(lds_addr(lds) + (uint32_t)wave * 1024u);
  L.sdst = __builtin_amdgcn_readfirstlane(lds_addr(lds) + C::DATA + (uint32_t)wave * 256u);
  MqLane o;
  {
    const int ra = wm * 128 + r32, rb = wn * 64 + r32;
    o.x = mq_swz(r32);
    o.a0 = ra * 128 + ((h ^ o.x) * 16);
    o.a1 = ra * 128 + (((2 + h) ^ o.x) * 16);
    o.b0 = 256 * 128 + rb * 128 + ((h ^ o.x) * 16);
    o.b1 = 256 * 128 + rb * 128 + (((2 + h) ^ o.x) * 16);
    o.sa = ra * 4 + h;
    o.sb = (256 + rb) * 4 + h;
  }
  // stream position v = tile v / nk, step v % nk
  qp_loader<EPI>(L, tl[0], A, As, B, Bs, N, K, ldb, bexp);
#pragma unroll
  for (int q = 0; q < C::OPS; ++q) mq_load<256>(L, q, 0u, 0);
  if (S > 1) {
    if (nk == 1) qp_loader<EPI>(L, tl[1], A, As, B, Bs, N, K, ldb, bexp);
#pragma unroll
    for (int q = 0; q < C::OPS; ++q) mq_load<256>(L, q, (uint32_t)(1 % nk) * 128u, 1);
  }
  vm_wait<0>();
  __builtin_amdgcn_s_barrier();
  MqFrags<256> F;
#pragma unroll
  for (int f = 0; f < 6; ++f) mq_read_one<256>(lds, 0, 0, o, f, F);
  v16f acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
  QpTile ct = tl[0];
  bool active = __builtin_amdgcn_readfirstlane((wm == 0 || ct.row_end - ct.row0 > 128) ? 1 : 0);
  for (int u = 0; u < S; ++u) {
    const int slot = u & 1, k = u % nk;
    mq_half<256>(L, lds, o, acc, F, slot, 1, false, 0u, 0, active);
    // own loads of step u+1 arrived; at a tile's first step the last tile's
    // stores came after them and are waited for too (a count that let them
    // stay in flight could release early: a store whose lanes are all out of
    // range need not hold its place in the count)
    vm_wait<0>();
    lgkm_wait0();
    __builtin_amdgcn_s_barrier();
    const int v = u + 2;
    const bool ld = v < S;
    if (ld && v % nk == 0) qp_loader<EPI>(L, tl[v / nk], A, As, B, Bs, N, K, ldb, bexp);
    const uint32_t kb = (uint32_t)(v % nk) * 128u;
    const int rslot = u + 1 < S ? slot ^ 1 : slot;
    mq_half<256>(L, lds, o, acc, F, rslot, 0, ld, kb, slot, active);
    if (EPI) {
      // the lane's row indices into prob (src[row], or row) at the tile's
      // first step, the probabilities at its second (each load waited by
      // the next step's barrier; with fewer steps, before the epilogue)
      if (k == 0) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int row = min(ct.row0 + wm * 128 + 32 * i + r32, ct.row_end - 1);
          pidx[i] = ep.src ? ep.src[row] : row;
        }
        if (nk == 1) vm_wait<0>();
      }
      if (k == min(1, nk - 1)) {
#pragma unroll
        for (int i = 0; i < 4; ++i) pr[i] = ep.prob[pidx[i]];
      }
    }
    if (k == nk - 1) {
      if (EPI) {
        if (nk <= 2) vm_wait<0>();
        qp_swiglu_store(acc, pr, rs, rss, ct, N / 2);
      } else {
        qp_store<OUT_F32>(acc, rs, ct, N, bias ? bias + (int64_t)ct.g * N : nullptr);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
      if (u + 1 < S) {
        ct = tl[(u + 1) / nk];
        active = __builtin_amdgcn_readfirstlane((wm == 0 || ct.row_end - ct.row0 > 128) ? 1 : 0);
      }
    }
  }
  vm_wait<0>();  // stores done and no load still targets this workgroup's LDS
}

// The gate_up grouped GEMM with the fused epilogue on the persistent kernel
// (N = 2 I, I % 128 == 0): q [M, I] E4M3, s [M, I / 32] E8M0.
__global__ __launch_bounds__(512, 1) void k_gemm_mxfp8_qp_swiglu(
    const uint8_t *__restrict__ A, const uint8_t *__restrict__ As,
    const uint8_t *__restrict__ B, const uint8_t *__restrict__ Bs,
    const int64_t *__restrict__ offsets, int64_t G, int64_t N, int64_t K, int64_t ntn,
    uint32_t q_bytes, SwigluEpi ep) {
  k_gemm_mxfp8_qp_body<false, true>(A, As, B, Bs, offsets, G, N, K, ntn, K, N * K, nullptr,
                                    q_bytes, ep, nullptr);
}

// The gate_up grouped GEMM with the fused epilogue: D = SwiGLU(C) x prob
// encoded as MXFP8 (C itself is never written).  N = 2 I, I % 128 == 0.
__global__ __launch_bounds__(256, 1) void k_gemm_mxfp8_swiglu(
    const uint8_t *__restrict__ A, const uint8_t *__restrict__ As,
    const uint8_t *__restrict__ B, const uint8_t *__restrict__ Bs,
    const int64_t *__restrict__ offsets, int64_t G, int64_t N, int64_t K, int64_t ntn,
    SwigluEpi ep) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[Mx3<256>::LDS];
  __shared__ int64_t sh[4];
  TileInfo ti;
  if (!lookup_row_tile<256, 256>(offsets, G, ntn, ti, sh)) return;
  if (ti.row_end - ti.row0 <= 128)
    mx3_tile<false, 128, true>(A, As, B, Bs, N, K, K, N * K, ti, lds, nullptr, &ep);
  else
    mx3_tile<false, 256, true>(A, As, B, Bs, N, K, K, N * K, ti, lds, nullptr, &ep);
}

// ------------------------------------------------------- MXFP8 weight grad
// Y_g[n, k] = sum over the group's tokens m of A[m, n] B[m, k], from the
// column-wise (32 x 1 block) MXFP8 copies stored transposed: At [N, M] with
// scale bytes Ats [N, M / 32], Bt [K, M] with Bts [K, M / 32] ([BW] MXFP8
// training: the backward GEMMs take the column-wise copies).  Each group's
// token range starts on a 32-token block boundary (per-expert padding), so
// blocks never straddle two experts.  One workgroup computes one 256 x 256
// tile of one Y_g with the forward's three-slot pipeline, in passes of up to
// 2048 tokens (the scale area holds 64 bytes per row): per pass the scale
// bytes are gathered through registers (the pass may start on any block, so
// the dword loads are realigned with a byte shift), chunks of 16 tokens past
// the group's end read zeros, and their blocks get the scale byte 127 (1.0)
// so that the zeros stay zeros.

__device__ uint4 g_mx_zero[1];

// Request step kt of a pass; `lim` = tokens in the pass.  Only the last two
// steps of a pass can reach past it (passes are padded to 128 tokens).
template <int TM>
__device__ __forceinline__ void mx3w_issue(const Mx3Src<TM> &L, const uint32_t (&lim_a)[Mx3<TM>::CA],
                                           const uint32_t (&lim_b)[Mx3<TM>::CB], int kt, int nk,
                                           int slot) {
  using C = Mx3<TM>;
  if (kt < nk - 2) {
    mx3_issue<TM>(L, kt, slot);
    return;
  }
  const uint32_t kb = (uint32_t)kt * 64u;
  const uint32_t base = L.dst + (uint32_t)slot * C::SLOT;
  const uint8_t *zero = reinterpret_cast<const uint8_t *>(g_mx_zero);
#pragma unroll
  for (int i = 0; i < C::CA; ++i)
    dma16(kb < lim_a[i] ? L.Ab + (L.oa[i] + kb) : zero, base + i * 4096);
#pragma unroll
  for (int i = 0; i < C::CB; ++i)
    dma16(kb < lim_b[i] ? L.Bb + (L.ob[i] + kb) : zero, base + TM * 64 + i * 4096);
}

// Scale bytes of one staged row for a pass: nb valid blocks starting at
// byte p (any alignment) of an array whose last byte is at `last`; blocks
// nb .. 4 dpr - 1 get 127.  Loaded as the 17 aligned dwords that cover them
// (clamped to the array), realigned by a byte shift, written dword-major as
// mx3_read expects.
__device__ __forceinline__ void mx3w_scales_row(const uint8_t *p, const uint8_t *last, int nb,
                                                int dpr, uint8_t *area, int row) {
  const uintptr_t a0 = (uintptr_t)p & ~(uintptr_t)3, amax = (uintptr_t)last & ~(uintptr_t)3;
  const uint32_t sh = (uint32_t)((uintptr_t)p & 3);
  uint32_t w[17];
#pragma unroll
  for (int j = 0; j < 17; ++j) {
    const uintptr_t aj = a0 + 4 * (uintptr_t)min(j, dpr);
    w[j] = *reinterpret_cast<const uint32_t *>(aj < amax ? aj : amax);
  }
  uint32_t *dst = reinterpret_cast<uint32_t *>(area) + (row >> 4) * dpr * 16 + (row & 15);
#pragma unroll
  for (int d = 0; d < 16; ++d) {
    if (d < dpr) {
      uint32_t v = __builtin_amdgcn_alignbyte(w[d + 1], w[d], sh);
      const int vb = nb - 4 * d;  // valid bytes of this dword (may be <= 0 or >= 4)
      if (vb < 4) {
        const uint32_t keep = vb <= 0 ? 0u : (0xFFFFFFFFu >> (8 * (4 - vb)));
        v = (v & keep) | (0x7F7F7F7Fu & ~keep);
      }
      dst[d * 16] = v;
    }
  }
}

template <bool OUT_F32>
__global__ __launch_bounds__(256, 1) void k_gemm_mxfp8_wgrad(
    const uint8_t *__restrict__ At, const uint8_t *__restrict__ Ats,
    const uint8_t *__restrict__ Bt, const uint8_t *__restrict__ Bts,
    const int64_t *__restrict__ offsets, int64_t G, int64_t M, int64_t N, int64_t K,
    int64_t ntm, int64_t ntn, void *__restrict__ out) {
  constexpr int TM = 256;
  using C = Mx3<TM>;
  constexpr int FI = C::FI, FJ = C::FJ, TN = C::TN, PASS = 32 * C::MAX_KS;
  __shared__ __attribute__((aligned(16))) uint8_t lds[C::LDS];
  // tiles of one expert are consecutive; workgroup b runs on XCD b % 8, so
  // an expert's tiles spread over all XCDs (expert loads are skewed)
  const int64_t total = G * ntm * ntn;
  const int64_t T = blockIdx.x;
  if (T >= total) return;
  const int64_t g = T / (ntm * ntn), rem = T - g * ntm * ntn;
  const int64_t n0 = (rem / ntn) * TM, k0 = (rem % ntn) * TN;
  const int64_t m0 = offsets[g], m1 = offsets[g + 1];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1, h = lane >> 5, r32 = lane & 31;
  const int rows_a = (int)min(N - n0, (int64_t)TM), rows_b = (int)min(K - k0, (int64_t)TN);
  const uint32_t Mu = (uint32_t)M;
  const int64_t MS = M / 32;

  v16f acc[FI][FJ];
#pragma unroll
  for (int i = 0; i < FI; ++i)
#pragma unroll
    for (int j = 0; j < FJ; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  Mx3Src<TM> L;
  L.dst = __builtin_amdgcn_readfirstlane(lds_addr(lds) + (uint32_t)wave * 1024u);
  int ka[C::CA], kb4[C::CB];  // logical 16-token chunk of each requested chunk
#pragma unroll
  for (int i = 0; i < C::CA; ++i) {
    const int c = tid + 256 * i, r = c >> 2, k = (c & 3) ^ ((r >> 2) & 3);
    L.oa[i] = (uint32_t)min(r, rows_a - 1) * Mu + 16u * k;
    ka[i] = 16 * k;
  }
#pragma unroll
  for (int i = 0; i < C::CB; ++i) {
    const int c = tid + 256 * i, r = c >> 2, k = (c & 3) ^ ((r >> 2) & 3);
    L.ob[i] = (uint32_t)min(r, rows_b - 1) * Mu + 16u * k;
    kb4[i] = 16 * k;
  }
  const uint8_t *lastA = Ats + N * MS - 1, *lastB = Bts + K * MS - 1;
  uint8_t *area = lds + C::NSLOT * C::SLOT;

  for (int64_t c0 = m0; c0 < m1; c0 += PASS) {
    const int len = (int)min((int64_t)PASS, m1 - c0);
    const int nk = 2 * ((len + 127) / 128);  // even, >= 2
    const int KS = 2 * nk, dpr = KS / 4;
    if (c0 != m0) __syncthreads();  // every wave is done with the last pass's LDS
    L.Ab = At + n0 * M + c0;
    L.Bb = Bt + k0 * M + c0;
    uint32_t lim_a[C::CA], lim_b[C::CB];
#pragma unroll
    for (int i = 0; i < C::CA; ++i) lim_a[i] = (uint32_t)max(len - ka[i], 0);
#pragma unroll
    for (int i = 0; i < C::CB; ++i) lim_b[i] = (uint32_t)max(len - kb4[i], 0);
    {
      const int nb = len / 32;
      const int64_t blk0 = c0 / 32;
      mx3w_scales_row(Ats + (n0 + min(tid, rows_a - 1)) * MS + blk0, lastA, nb, dpr, area, tid);
      mx3w_scales_row(Bts + (k0 + min(tid, rows_b - 1)) * MS + blk0, lastB, nb, dpr, area,
                      TM + tid);
    }
    Mx3Lane o;
    {
      const int ra = wm * (TM / 2) + r32, rb = wn * 128 + r32;
      o.a_lo = mx3_off(ra, h);
      o.a_hi = mx3_off(ra, 2 + h);
      o.b_lo = TM * 64 + mx3_off(rb, h);
      o.b_hi = TM * 64 + mx3_off(rb, 2 + h);
      o.sa = (ra >> 4) * KS * 16 + (ra & 15) * 4;
      o.sb = ((TM + rb) >> 4) * KS * 16 + ((TM + rb) & 15) * 4;
      o.ks = KS;
    }
    mx3w_issue<TM>(L, lim_a, lim_b, 0, nk, 0);
    mx3w_issue<TM>(L, lim_a, lim_b, 1, nk, 1);
    mx3w_issue<TM>(L, lim_a, lim_b, min(2, nk - 1), nk, 2);
    vm_wait<2 * C::OPS>();  // step 0
    lgkm_wait0();           // this wave's scale bytes are in LDS
    __builtin_amdgcn_s_barrier();
    Mx3Frags<TM> F0, F1;
    mx3_read<TM>(lds, 0, 0, o, F0);
    int slot = 0;
    for (int kt = 0; kt < nk; kt += 2) {
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const int k = kt + half;
        // chunks past the pass read the zero line (only the last two steps
        // of a pass can reach past it)
        mx3_step_with<TM>(L, lds, o, k, nk, slot, acc, half ? F1 : F0, half ? F0 : F1,
                          [&](int q, uint32_t kb) {
                            const uint8_t *zero = reinterpret_cast<const uint8_t *>(g_mx_zero);
                            return q < C::CA
                                       ? (kb < lim_a[q] ? L.Ab + (L.oa[q] + kb) : zero)
                                       : (kb < lim_b[q - C::CA] ? L.Bb + (L.ob[q - C::CA] + kb)
                                                                : zero);
                          });
        slot = slot == 2 ? 0 : slot + 1;
      }
    }
    vm_wait<0>();  // no load may still target this workgroup's LDS
  }
  const int64_t esz = OUT_F32 ? 4 : 2;
  void *og = static_cast<uint8_t *>(out) + g * N * K * esz;
#pragma unroll
  for (int i = 0; i < FI; ++i)
#pragma unroll
    for (int j = 0; j < FJ; ++j)
      mx3_store<OUT_F32>(acc[i][j], og, K, n0, N, k0, wm * (TM / 2) + 32 * i, wn * 128 + 32 * j);
}

// ------------------------------------ MXFP8 weight grad, persistent kernel
// dW_g = dY_g^T X_g as k_gemm_mxfp8_wgrad computes it, on the eight-wave
// ring of k_gemm_mxfp8_qp: one workgroup per CU runs a sequence of 256 x 256
// tiles (g, n-tile, k-tile) as one stream of 128-token steps (a tile takes
// ceil(len / 128) steps over its expert's len tokens, an empty expert's tile
// one step of zeros), and each tile's output leaves by buffer stores that
// drain under the next tile's steps.
// Work per tile grows with the expert's tokens (a skewed routing puts 7444
// of 65536 rows in one expert of 128), so the tiles are ordered by expert,
// heaviest first (each workgroup ranks the experts by their step counts),
// and handed out as a list schedule: workgroup w starts with tile w, then,
// with a counter in the caller's workspace, takes the next unclaimed tile
// whenever it starts one (fetched three tiles ahead, so its value is back
// before it is needed); without a workspace the tiles are dealt in
// alternating directions (w, 2P - 1 - w, 2P + w, ...).  Workgroups of one XCD
// have consecutive ranks w, so the first tiles of an expert share an L2.
// Operands come in by buffer loads into LDS: chunks at or past the expert's
// last token, and rows past N or K, take an offset beyond the buffer and the
// hardware writes zeros for them.  A step's four E8M0 bytes of a row start
// at byte m0 / 32 + 4 k of the row's scales, in general not on a 4-byte
// boundary, so each row brings the two aligned words that hold them (8
// bytes per row in the slot) and the reader takes its byte at the row's
// shift.  The tail blocks read whatever scale bytes follow (another expert's,
// valid E8M0 values) against zero data.
struct Mw {
  static constexpr int ROWS = 512;
  static constexpr int DATA = ROWS * 128;
  static constexpr int SLOT = DATA + ROWS * 8;
  static constexpr int NSLOT = 2, LDS = NSLOT * SLOT;
  static constexpr int CA = 4, CB = 4, OPS = CA + CB + 2;
};
static_assert(Mw::DATA == Mq<256>::DATA, "the forward ring's data layout");

constexpr int MW_MAXG = 512;  // experts (the per-expert tables live in LDS)

struct MwTile {
  int32_t g, n0, k0, m0, len;
};

typedef __attribute__((address_space(3))) void lds_void_t;

__device__ __forceinline__ lds_void_t *lds_ptr(uint32_t a) {
  return reinterpret_cast<lds_void_t *>((uintptr_t)a);
}

struct MwSrc {
  __amdgpu_buffer_rsrc_t ra, rb, rsa, rsb;  // At, Bt, Ats, Bts
  uint32_t oa[4], ob[4];  // lane's chunk offsets at step 0 (QP_OOB: row past N or K)
  uint32_t sa, sb;        // lane's aligned scale word at step 0 (QP_OOB likewise)
  uint32_t tc;            // token offset of the lane's chunk within a step
  int32_t len;            // tokens of the tile's expert
  uint32_t dst, sdst;     // LDS addresses of slot 0 for this wave's lanes
};

// Offsets of tile t: load q (0..3) of lane tid brings row 64 q + tid / 8 of
// the A and of the B panel, physical chunk tid % 8 = logical chunk
// (tid % 8) ^ mq_swz(row) = (tid % 8) ^ (tid / 16 % 8) (the ring's swizzle),
// so every load of a lane covers
// the same 16 tokens tc .. tc + 15 of a step.  Scale word op 0 brings word
// tid % 2 of A row tid / 2, op 1 the same of B row tid / 2.
__device__ __forceinline__ void mw_loader(MwSrc &L, const MwTile &t, int64_t M, int64_t N,
                                          int64_t K) {
  const int tid = threadIdx.x;
  const uint32_t Mu = (uint32_t)M, MS = (uint32_t)(M / 32);
  const uint32_t c16 = 16u * (uint32_t)((tid & 7) ^ ((tid >> 4) & 7));
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int r = 64 * q + (tid >> 3);
    L.oa[q] = t.n0 + r < N ? (uint32_t)(t.n0 + r) * Mu + (uint32_t)t.m0 + c16 : QP_OOB;
    L.ob[q] = t.k0 + r < K ? (uint32_t)(t.k0 + r) * Mu + (uint32_t)t.m0 + c16 : QP_OOB;
  }
  const int r = tid >> 1;
  const uint32_t w = 4u * (uint32_t)(tid & 1), b0 = (uint32_t)t.m0 / 32u;
  L.sa = t.n0 + r < N ? (((uint32_t)(t.n0 + r) * MS + b0) & ~3u) + w : QP_OOB;
  L.sb = t.k0 + r < K ? (((uint32_t)(t.k0 + r) * MS + b0) & ~3u) + w : QP_OOB;
  L.len = t.len;
}

// Load q of step kt (chunks 0..3 of A, 0..3 of B, the A and the B scale
// words) into `slot`.
__device__ __forceinline__ void mw_load(const MwSrc &L, int q, int kt, int slot) {
  const uint32_t sl = (uint32_t)slot * Mw::SLOT, kb = (uint32_t)kt * 128u;
  const bool in = kb + L.tc < (uint32_t)L.len;
  if (q < 4) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(L.ra, lds_ptr(L.dst + sl + q * 8192),
                                             16, (int)(in ? L.oa[q] + kb : QP_OOB), 0, 0, 0);
  } else if (q < 8) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(L.rb, lds_ptr(L.dst + sl + 32768 + (q - 4) * 8192),
                                             16, (int)(in ? L.ob[q - 4] + kb : QP_OOB), 0, 0, 0);
  } else if (q == 8) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(L.rsa, lds_ptr(L.sdst + sl), 4,
                                             (int)(L.sa + 4u * (uint32_t)kt), 0, 0, 0);
  } else {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(L.rsb, lds_ptr(L.sdst + sl + 2048), 4,
                                             (int)(L.sb + 4u * (uint32_t)kt), 0, 0, 0);
  }
}

// As mq_read_one with 8 scale bytes per row: o.sa / o.sb include the row's
// shift, which is the same for rows 32 apart (32 MS is a multiple of 4).
__device__ __forceinline__ void mw_read_one(const uint8_t *lds, int slot, int half,
                                            const MqLane &o, int f, MqFrags<256> &F) {
  const uint8_t *cur = lds + slot * Mw::SLOT;
  const int hx = half * 64;
  if (f < 4) {
    F.a[f] = mw_frag(cur + (o.a0 ^ hx) + 4096 * f, cur + (o.a1 ^ hx) + 4096 * f);
    F.sa[f] = cur[Mw::DATA + o.sa + 2 * half + 256 * f];
  } else {
    const int g = f - 4;
    F.b[g] = mw_frag(cur + (o.b0 ^ hx) + 4096 * g, cur + (o.b1 ^ hx) + 4096 * g);
    F.sb[g] = cur[Mw::DATA + o.sb + 2 * half + 256 * g];
  }
}

// One K-half (as mq_half): 8 MFMAs, the loads of step lk into lslot spread
// over them, each fragment replaced by fragment f of (rslot, rhalf).
__device__ __forceinline__ void mw_half(const MwSrc &L, const uint8_t *lds, const MqLane &o,
                                        v16f (&acc)[4][2], MqFrags<256> &F, int rslot,
                                        int rhalf, bool loads, int lk, int lslot, bool MF) {
#pragma unroll
  for (int m = 0; m < 8; ++m) {
    const int j = m / 4, i = m % 4;
    if (MF)
      acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(F.b[j], F.a[i], acc[i][j], 0,
                                                                   0, 0, F.sb[j], 0, F.sa[i]);
    if (loads) {
#pragma unroll
      for (int q = 2 * m; q < 2 * m + 2 && q < Mw::OPS; ++q) mw_load(L, q, lk, lslot);
    }
    if (m == 3) mw_read_one(lds, rslot, rhalf, o, 4, F);      // b0
    if (m >= 4) mw_read_one(lds, rslot, rhalf, o, i, F);      // a_i
    if (m == 7) mw_read_one(lds, rslot, rhalf, o, 5, F);      // b1
    __builtin_amdgcn_sched_barrier(0);
  }
}

__device__ __forceinline__ int mw_steps(int32_t len) { return len > 0 ? (len + 127) / 128 : 1; }

// The reader's scale byte offsets for tile t: row shift of A row wm 128 + r
// and of B row wn 64 + r.
__device__ __forceinline__ void mw_shifts(MqLane &o, const MwTile &t, int64_t M) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 2, wn = wave & 3, h = lane >> 5, r32 = lane & 31;
  const uint32_t MS = (uint32_t)(M / 32), b0 = (uint32_t)t.m0 / 32u;
  const int ra = wm * 128 + r32, rb = wn * 64 + r32;
  const uint32_t sha = ((uint32_t)(t.n0 + ra) * MS + b0) & 3u;
  const uint32_t shb = ((uint32_t)(t.k0 + rb) * MS + b0) & 3u;
  o.sa = ra * 8 + (int)sha + h;
  o.sb = (256 + rb) * 8 + (int)shb + h;
}

template <bool OUT_F32, bool DYN>
__global__ __launch_bounds__(512, 1) void k_gemm_mxfp8_wgrad_qp(
    const uint8_t *__restrict__ At, const uint8_t *__restrict__ Ats,
    const uint8_t *__restrict__ Bt, const uint8_t *__restrict__ Bts,
    const int64_t *__restrict__ offsets, int32_t G, int64_t M, int64_t N, int64_t K,
    int32_t ntm, int32_t ntn, void *__restrict__ out, uint32_t *__restrict__ ctr) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[Mw::LDS];
  __shared__ int32_t e_ord[MW_MAXG], e_m0[MW_MAXG], e_len[MW_MAXG];
  __shared__ int32_t seq[4];  // DYN: tile j of this workgroup's sequence at j % 4
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 2, wn = wave & 3, h = lane >> 5, r32 = lane & 31;

  // ---- experts ranked by steps, descending (ties by index)
  int32_t *stp = reinterpret_cast<int32_t *>(lds);  // setup only, before any ring load
  for (int g = tid; g < G; g += 512) {
    const int32_t m0 = (int32_t)offsets[g], len = (int32_t)(offsets[g + 1] - offsets[g]);
    e_m0[g] = m0;
    e_len[g] = len;
    stp[g] = mw_steps(len);
  }
  __syncthreads();
  for (int g = tid; g < G; g += 512) {
    const int32_t s = stp[g];
    int rank = 0;
    for (int e = 0; e < G; ++e) {
      const int32_t se = stp[e];
      rank += (se > s || (se == s && e < g)) ? 1 : 0;
    }
    e_ord[rank] = g;
  }
  const int32_t per_g = ntm * ntn, total = G * per_g;
  const int32_t P = (int32_t)gridDim.x;
  const int32_t w = (int32_t)(blockIdx.x % 8) * (P / 8) + (int32_t)(blockIdx.x / 8);
  if (DYN && tid == 0) {  // tiles 1 .. 3 of the sequence; later ones three ahead
#pragma unroll
    for (int j = 1; j < 4; ++j)
      seq[j] = P + (int32_t)__hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED,
                                                   __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();  // tables and seq published; stp is no longer read
  auto tile_at = [&](int j) -> int32_t {  // tau of the j-th tile of this workgroup
    if (j == 0) return w;
    if (DYN) return seq[j & 3];
    return j * P + ((j & 1) ? P - 1 - w : w);
  };
  auto tile_of = [&](int32_t tau) -> MwTile {
    const int32_t e = e_ord[tau / per_g], rem = tau % per_g;
    return MwTile{e, (rem / ntn) * 256, (rem % ntn) * 256, e_m0[e], e_len[e]};
  };
  if (w >= total) return;

  const int64_t esz = OUT_F32 ? 4 : 2;
  MwSrc L;
  L.ra = __builtin_amdgcn_make_buffer_rsrc((void *)At, (short)0, (int)(N * M), 0x00020000);
  L.rb = __builtin_amdgcn_make_buffer_rsrc((void *)Bt, (short)0, (int)(K * M), 0x00020000);
  L.rsa = __builtin_amdgcn_make_buffer_rsrc((void *)Ats, (short)0, (int)(N * (M / 32)), 0x00020000);
  L.rsb = __builtin_amdgcn_make_buffer_rsrc((void *)Bts, (short)0, (int)(K * (M / 32)), 0x00020000);
  L.tc = 16u * (uint32_t)((tid & 7) ^ ((tid >> 4) & 7));
  L.dst = __builtin_amdgcn_readfirstlane(lds_addr(lds) + (uint32_t)wave * 1024u);
  L.sdst = __builtin_amdgcn_readfirstlane(lds_addr(lds) + Mw::DATA + (uint32_t)wave * 256u);
  MqLane o;
  {
    const int ra = wm * 128 + r32, rb = wn * 64 + r32;
    o.x = mq_swz(r32);
    o.a0 = ra * 128 + ((h ^ o.x) * 16);
    o.a1 = ra * 128 + (((2 + h) ^ o.x) * 16);
    o.b0 = 256 * 128 + rb * 128 + ((h ^ o.x) * 16);
    o.b1 = 256 * 128 + rb * 128 + (((2 + h) ^ o.x) * 16);
  }

  // current step: tile ci (ct), step ck of cn; load cursor, two positions
  // ahead: tile vi, step vk of vn, vok while that tile exists (L holds its
  // offsets)
  int ci = 0, ck = 0;
  MwTile ct = tile_of(w);
  int cn = mw_steps(ct.len);
  mw_shifts(o, ct, M);
  int vi = 0, vk = 0, vn = cn;
  bool vok = true;
  mw_loader(L, ct, M, N, K);
#pragma unroll
  for (int q = 0; q < Mw::OPS; ++q) mw_load(L, q, 0, 0);
  auto advance = [&]() {
    if (++vk == vn) {
      vk = 0;
      ++vi;
      const int32_t tau = tile_at(vi);
      vok = tau < total;
      if (vok) {
        const MwTile t = tile_of(tau);
        vn = mw_steps(t.len);
        mw_loader(L, t, M, N, K);
      }
    }
  };
  advance();
  if (vok) {
#pragma unroll
    for (int q = 0; q < Mw::OPS; ++q) mw_load(L, q, vk, 1);
    advance();
  }
  vm_wait<0>();
  __builtin_amdgcn_s_barrier();
  MqFrags<256> F;
#pragma unroll
  for (int f = 0; f < 6; ++f) mw_read_one(lds, 0, 0, o, f, F);
  v16f acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
  bool active = __builtin_amdgcn_readfirstlane((wm == 0 || ct.n0 + 128 < N) ? 1 : 0);
  uint32_t fetched = 0;  // DYN, thread 0: a counter value on its way back
  bool pend = false;
  for (int u = 0;; ++u) {
    const int slot = u & 1;
    mw_half(L, lds, o, acc, F, slot, 1, false, 0, 0, active);
    // own loads of step u+1 arrived (at a tile's first step after the last
    // tile's stores, which are waited for too: only loads keep their order
    // in the count)
    vm_wait<0>();
    if (DYN && pend) {  // (thread 0 only) tile ci + 3 of the sequence
      seq[(ci + 3) & 3] = P + (int32_t)fetched;
      pend = false;
    }
    lgkm_wait0();
    __builtin_amdgcn_s_barrier();
    const bool last = ck == cn - 1;
    int32_t tau_n = 0;
    bool more = !last;
    if (last) {
      tau_n = tile_at(ci + 1);
      more = tau_n < total;
      if (more) mw_shifts(o, tile_of(tau_n), M);  // the reads below are step u+1's
    }
    const bool ld = vok;
    mw_half(L, lds, o, acc, F, more ? slot ^ 1 : slot, 0, ld, vk, slot, active);
    if (ld) advance();
    if (!last) {
      ++ck;
      continue;
    }
    if (DYN && more && tid == 0) {
      // claim tile ci + 4, the next tile's third successor (written at the
      // next step); issued before the stores, so that waiting for it does
      // not wait for them
      fetched = __builtin_amdgcn_atomic_inc32(ctr, 0xFFFFFFFFu, __ATOMIC_RELAXED, "agent");
      pend = true;
    }
    {
      const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
          static_cast<uint8_t *>(out) + (int64_t)ct.g * N * K * esz, (short)0,
          (int)(N * K * esz), 0x00020000);
      qp_store<OUT_F32>(acc, rs, QpTile{ct.n0, (int32_t)N, ct.g, ct.k0}, K);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
    if (!more) break;
    ++ci;
    ct = tile_of(tau_n);
    cn = mw_steps(ct.len);
    ck = 0;
    active = __builtin_amdgcn_readfirstlane((wm == 0 || ct.n0 + 128 < N) ? 1 : 0);
  }
  vm_wait<0>();  // stores done and no load still targets this workgroup's LDS
}

// Clears the tile counter of the dynamic weight-gradient schedule.
__global__ void k_zero_u32(uint32_t *p) { p[0] = 0u; }

// ----------------------------------------------------- block-scaled FP8
// DeepSeek-V3-style operands ("Towards Blackwell-Native 8-bit and 4-bit RL",
// Why Blackwell-native recipes: 1 x 128 activation tiles and 128 x 128 weight
// blocks with FP32 scales, applied in software around the matrix core):
//   Y[m, n] = sum over 128-K blocks kb of sa[m, kb] sb[n / 128, kb]
//             (sum over k in kb of qa[m, k] qb[n, k]).
// The forward's ring and 128 x 256 tiles; each 128-K block's products go
// into a fresh accumulator through the FP8 matrix core (hardware scales
// fixed at 2^0), which is then added into the result times the product of
// the two binary32 scales.  All scales of the tile are preloaded to LDS:
// sa as [kb][row], sb as [column block][kb].

constexpr int FB_MAX_KB = 64;  // K <= 8192
constexpr int FB_TM = 128;
constexpr int FB_AREA = 256 * ((FB_TM * FB_MAX_KB + 2 * FB_MAX_KB + 255) / 256);  // dwords

__device__ __forceinline__ void fb_read(const uint8_t *lds, int slot, const Mx3Lane &o,
                                        Mx3Frags<FB_TM> &F) {
  using C = Mx3<FB_TM>;
  const uint8_t *cur = lds + slot * C::SLOT;
#pragma unroll
  for (int i = 0; i < C::FI; ++i) {
    const uint4 lo = *reinterpret_cast<const uint4 *>(cur + o.a_lo + 2048 * i);
    const uint4 hi = *reinterpret_cast<const uint4 *>(cur + o.a_hi + 2048 * i);
    F.a[i] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
  }
#pragma unroll
  for (int j = 0; j < C::FJ; ++j) {
    const uint4 lo = *reinterpret_cast<const uint4 *>(cur + o.b_lo + 2048 * j);
    const uint4 hi = *reinterpret_cast<const uint4 *>(cur + o.b_hi + 2048 * j);
    F.b[j] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
  }
}

template <bool FIRST>
__device__ __forceinline__ void fb_mma(const Mx3Frags<FB_TM> &F,
                                       v16f (&part)[Mx3<FB_TM>::FI][Mx3<FB_TM>::FJ]) {
  const v16f zero = {};
#pragma unroll
  for (int j = 0; j < Mx3<FB_TM>::FJ; ++j)
#pragma unroll
    for (int i = 0; i < Mx3<FB_TM>::FI; ++i)
      part[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
          F.b[j], F.a[i], FIRST ? zero : part[i][j], 0, 0, 0, 127, 0, 127);
}

template <bool FIRST>
__device__ __forceinline__ void fb_step(const Mx3Src<FB_TM> &L, const uint8_t *lds,
                                        const Mx3Lane &o, int kt, int nk, int slot,
                                        v16f (&part)[Mx3<FB_TM>::FI][Mx3<FB_TM>::FJ],
                                        const Mx3Frags<FB_TM> &cur, Mx3Frags<FB_TM> &next) {
  vm_wait<Mx3<FB_TM>::OPS>();
  lgkm_wait0();
  __builtin_amdgcn_s_barrier();
  mx3_issue<FB_TM>(L, min(kt + 3, nk - 1), slot);
  __builtin_amdgcn_sched_barrier(0);
  fb_read(lds, slot == 2 ? 0 : slot + 1, o, next);
  __builtin_amdgcn_sched_barrier(0);
  fb_mma<FIRST>(cur, part);
}

template <bool OUT_F32, bool BIAS>
__global__ __launch_bounds__(256, 1) void k_gemm_fp8_block(
    const uint8_t *__restrict__ A, const float *__restrict__ As, const uint8_t *__restrict__ B,
    const float *__restrict__ Bs, const int64_t *__restrict__ offsets, int64_t G, int64_t N,
    int64_t K, int64_t ntn, void *__restrict__ out, const float *__restrict__ bias) {
  constexpr int TM = FB_TM;
  using C = Mx3<TM>;
  constexpr int FI = C::FI, FJ = C::FJ, TN = C::TN;
  __shared__ __attribute__((aligned(16))) uint8_t lds[C::NSLOT * C::SLOT + 4 * FB_AREA];
  __shared__ int64_t sh[4];
  TileInfo ti;
  if (!lookup_row_tile<256, TM>(offsets, G, ntn, ti, sh)) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1, h = lane >> 5, r32 = lane & 31;
  const int KB = (int)(K / 128);
  const uint32_t Ku = (uint32_t)K;
  const int rows_a = (int)min(ti.row_end - ti.row0, (int64_t)TM);
  const int rows_b = (int)min(N - ti.n0, (int64_t)TN);
  Mx3Src<TM> L;
  L.Ab = A + ti.row0 * K;
  L.Bb = B + (ti.g * N + ti.n0) * K;
  L.dst = __builtin_amdgcn_readfirstlane(lds_addr(lds) + (uint32_t)wave * 1024u);
#pragma unroll
  for (int i = 0; i < C::CA; ++i) {
    const int c = tid + 256 * i, r = c >> 2, k = (c & 3) ^ ((r >> 2) & 3);
    L.oa[i] = (uint32_t)min(r, rows_a - 1) * Ku + 16u * k;
  }
#pragma unroll
  for (int i = 0; i < C::CB; ++i) {
    const int c = tid + 256 * i, r = c >> 2, k = (c & 3) ^ ((r >> 2) & 3);
    L.ob[i] = (uint32_t)min(r, rows_b - 1) * Ku + 16u * k;
  }
  Mx3Lane o;
  {
    const int ra = wm * (TM / 2) + r32, rb = wn * 128 + r32;
    o.a_lo = mx3_off(ra, h);
    o.a_hi = mx3_off(ra, 2 + h);
    o.b_lo = TM * 64 + mx3_off(rb, h);
    o.b_hi = TM * 64 + mx3_off(rb, 2 + h);
    o.sa = o.sb = o.ks = 0;
  }
  // scales: dword d < TM KB is sa of row d % TM, block d / TM; the next 2 KB
  // are sb of the tile's two 128-column blocks (a block past N repeats the
  // first; its results are not stored)
  const float *sa_l = reinterpret_cast<const float *>(lds + C::NSLOT * C::SLOT);
  const float *sb_l = sa_l + TM * KB;
  {
    const uint32_t sbase = __builtin_amdgcn_readfirstlane(lds_addr(sa_l) + (uint32_t)wave * 256u);
    const int total = TM * KB + 2 * KB, nq = (total + 255) / 256;
    const int64_t nb0 = (ti.g * N + ti.n0) / 128;
    for (int q = 0; q < nq; ++q) {
      const int d = min(256 * q + tid, total - 1);
      const float *src;
      if (d < TM * KB) {
        src = As + (ti.row0 + min(d % TM, rows_a - 1)) * (int64_t)KB + d / TM;
      } else {
        const int e = d - TM * KB, blk = e / KB;
        src = Bs + (nb0 + (ti.n0 + 128 * blk < N ? blk : 0)) * (int64_t)KB + e % KB;
      }
      dma4(src, sbase + 1024u * (uint32_t)q);
    }
  }

  v16f acc[FI][FJ], part[FI][FJ];
#pragma unroll
  for (int i = 0; i < FI; ++i)
#pragma unroll
    for (int j = 0; j < FJ; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  const int nk = (int)(K / 64);  // even, >= 2
  mx3_issue<TM>(L, 0, 0);
  mx3_issue<TM>(L, 1, 1);
  mx3_issue<TM>(L, min(2, nk - 1), 2);
  vm_wait<2 * C::OPS>();  // the scales and step 0
  __builtin_amdgcn_s_barrier();
  Mx3Frags<TM> F0, F1;
  fb_read(lds, 0, o, F0);
  int slot = 0;
  for (int kb = 0; kb < KB; ++kb) {
    const int kt = 2 * kb;
    fb_step<true>(L, lds, o, kt, nk, slot, part, F0, F1);
    slot = slot == 2 ? 0 : slot + 1;
    fb_step<false>(L, lds, o, kt + 1, nk, slot, part, F1, F0);
    slot = slot == 2 ? 0 : slot + 1;
    const float sbv = sb_l[wn * KB + kb];
#pragma unroll
    for (int i = 0; i < FI; ++i) {
      const float sc = sa_l[kb * TM + wm * (TM / 2) + 32 * i + r32] * sbv;
#pragma unroll
      for (int j = 0; j < FJ; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = fmaf(part[i][j][r], sc, acc[i][j][r]);
    }
  }
  vm_wait<0>();  // no load may still target this workgroup's LDS at exit
#pragma unroll
  for (int i = 0; i < FI; ++i)
#pragma unroll
    for (int j = 0; j < FJ; ++j)
      mx3_store<OUT_F32>(acc[i][j], out, N, ti.row0, ti.row_end, ti.n0, wm * (TM / 2) + 32 * i,
                         wn * 128 + 32 * j, BIAS ? bias + ti.g * N : nullptr);
}

// ------------------------------------------------------------------- BF16

// Stage a tile whose rows are contiguous in memory and whose contraction
// index is strided (element (r, k) at base[k * stride + r]) as [r][k] in
// LDS: 64 K x 128 rows of 16-bit values, transposed on the way.
struct RowContigLoader {
  uint4 v[4];
  __device__ void load(const uint16_t *__restrict__ base, int64_t stride, int64_t rows,
                       int64_t k0, int64_t kmax) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = threadIdx.x + 256 * i;  // 64 k x 16 chunks of 8 rows
      const int kk = c >> 4, rc = (c & 15) * 8;
      v[i] = make_uint4(0, 0, 0, 0);
      if (k0 + kk < kmax && rc < rows)
        v[i] = *reinterpret_cast<const uint4 *>(base + (k0 + kk) * stride + rc);
    }
  }
  __device__ void store(uint8_t *lds) const {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = threadIdx.x + 256 * i;
      const int kk = c >> 4, rc = (c & 15) * 8;
      const uint32_t w[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint16_t h = (uint16_t)(w[e >> 1] >> (16 * (e & 1)));
        *reinterpret_cast<uint16_t *>(lds + (rc + e) * GT_PITCH + kk * 2) = h;
      }
    }
  }
};

__device__ __forceinline__ v8bf frag_bf16(const uint8_t *lds, int row, int s) {
  const int lane = threadIdx.x & 63;
  const uint4 v = *reinterpret_cast<const uint4 *>(lds + row * GT_PITCH + 32 * s +
                                                   16 * (lane >> 5));
  return __builtin_bit_cast(v8bf, v);
}

// FPROP: A [M, K] k-contig, B [G, N, K] k-contig.
// DGRAD: A [M, K] k-contig, B [G, K, N] row-contig (B_ROW).
template <bool B_ROW, bool OUT_F32>
__global__ __launch_bounds__(256) void k_gemm_bf16_rows(
    const uint16_t *__restrict__ A, const uint16_t *__restrict__ B,
    const int64_t *__restrict__ offsets, int64_t G, int64_t N, int64_t K, int64_t ntn,
    void *__restrict__ out, const float *__restrict__ bias) {
  __shared__ __attribute__((aligned(16))) uint8_t lA[GT_M * GT_PITCH];
  __shared__ __attribute__((aligned(16))) uint8_t lB[GT_N * GT_PITCH];
  __shared__ int64_t sh[4];
  TileInfo ti;
  if (!lookup_row_tile(offsets, G, ntn, ti, sh)) return;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int64_t rows_a = ti.row_end - ti.row0;
  const int64_t rows_b = N - ti.n0;
  const uint8_t *Ab = reinterpret_cast<const uint8_t *>(A + ti.row0 * K);
  v16f acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
  KContigLoader la;
  KContigLoader lbk;
  RowContigLoader lbr;
  la.load(Ab, K * 2, rows_a, 0, K * 2);
  if (B_ROW)
    lbr.load(B + ti.g * K * N + ti.n0, N, rows_b, 0, K);
  else
    lbk.load(reinterpret_cast<const uint8_t *>(B + (ti.g * N + ti.n0) * K), K * 2, rows_b, 0,
             K * 2);
  const int KT = GT_KB / 2;  // 64 bf16 per step
  const int nk = (int)((K + KT - 1) / KT);
  for (int kt = 0; kt < nk; ++kt) {
    la.store(lA);
    if (B_ROW) lbr.store(lB); else lbk.store(lB);
    __syncthreads();
    if (kt + 1 < nk) {
      la.load(Ab, K * 2, rows_a, (int64_t)(kt + 1) * GT_KB, K * 2);
      if (B_ROW)
        lbr.load(B + ti.g * K * N + ti.n0, N, rows_b, (int64_t)(kt + 1) * KT, K);
      else
        lbk.load(reinterpret_cast<const uint8_t *>(B + (ti.g * N + ti.n0) * K), K * 2, rows_b,
                 (int64_t)(kt + 1) * GT_KB, K * 2);
    }
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      v8bf fa[2], fb[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        fa[i] = frag_bf16(lA, wm * 64 + 32 * i + (lane & 31), s);
        fb[i] = frag_bf16(lB, wn * 64 + 32 * i + (lane & 31), s);
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
      store_acc<OUT_F32>(acc[i][j], out, N, ti.row0, ti.row_end, ti.n0, N, wm * 64 + 32 * i,
                         wn * 64 + 32 * j, nullptr, 1.0f, bias ? bias + ti.g * N : nullptr);
}

// WGRAD: Y_g[n, k] = sum_{m in g} A[m, n] B[m, k]; A [M, N], B [M, K], both
// contraction-strided.  Tile = (group, n tile, k tile); contraction in steps
// of 64 rows of the group.
template <bool OUT_F32>
__global__ __launch_bounds__(256) void k_gemm_bf16_wgrad(
    const uint16_t *__restrict__ A, const uint16_t *__restrict__ B,
    const int64_t *__restrict__ offsets, int64_t N, int64_t K, int64_t ntn, int64_t ntk,
    void *__restrict__ out) {
  __shared__ __attribute__((aligned(16))) uint8_t lA[GT_M * GT_PITCH];
  __shared__ __attribute__((aligned(16))) uint8_t lB[GT_N * GT_PITCH];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int64_t t = blockIdx.x;
  const int64_t g = t / (ntn * ntk);
  const int64_t n0 = ((t / ntk) % ntn) * GT_M;
  const int64_t k0 = (t % ntk) * GT_N;
  const int64_t m0 = offsets[g], m1 = offsets[g + 1];
  const int64_t rows_a = N - n0, rows_b = K - k0;
  v16f acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
  RowContigLoader la, lb;
  const int KT = 64;
  const int64_t len = m1 - m0;
  const int nk = (int)((len + KT - 1) / KT);
  if (nk > 0) {
    la.load(A + m0 * N + n0, N, rows_a, 0, len);
    lb.load(B + m0 * K + k0, K, rows_b, 0, len);
  }
  for (int kt = 0; kt < nk; ++kt) {
    la.store(lA);
    lb.store(lB);
    __syncthreads();
    if (kt + 1 < nk) {
      la.load(A + m0 * N + n0, N, rows_a, (int64_t)(kt + 1) * KT, len);
      lb.load(B + m0 * K + k0, K, rows_b, (int64_t)(kt + 1) * KT, len);
    }
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      v8bf fa[2], fb[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        fa[i] = frag_bf16(lA, wm * 64 + 32 * i + (lane & 31), s);
        fb[i] = frag_bf16(lB, wn * 64 + 32 * i + (lane & 31), s);
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
    }
    __syncthreads();
  }
  void *o = OUT_F32 ? (void *)(static_cast<float *>(out) + g * N * K)
                    : (void *)(static_cast<uint16_t *>(out) + g * N * K);
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
      store_acc<OUT_F32>(acc[i][j], o, K, n0, N, k0, K, wm * 64 + 32 * i, wn * 64 + 32 * j);
}

// ---------------------------------------------- BF16, pipelined large tiles
//
// The MXFP8 pipeline above (3-slot ring of direct global->LDS loads, operands
// read one step ahead, 256 x 256 tiles with 128 x 128 per wave in AGPRs,
// transposed accumulators with 16-byte stores) carrying bf16 operands: a step
// is 32 contraction values, i.e. two v_mfma_f32_32x32x16_bf16 per fragment
// pair.  An operand is staged in one of two layouts of TM x 64 bytes:
//  * KL, contraction contiguous in memory (FPROP operands, DGRAD's tokens):
//    TM rows of 64 bytes, the MXFP8 ring's swizzle, 16-byte LDS reads;
//  * ML, contraction strided (DGRAD's weight, both WGRAD operands): 32
//    contraction rows of 256 outputs (512 bytes, 32 chunks of 16 bytes, chunk
//    x of row r stored at x ^ 4 f(r), f(r) = (r & 3) | ((r >> 3) & 1) << 2),
//    read with the gfx950 transposing LDS read ds_read_b64_tr_b16.  Within
//    each group of 16 lanes that read gives lane i, as its element e, element
//    i % 4 of the 8 bytes addressed by lane 4 e + i / 4 (measured); so lanes
//    4 r + c addressing row r, outputs 4 c .. 4 c + 3 of a 4-row x 16-output
//    block leave lane i with the 4 contraction values of output i.  Lanes
//    16 q + j read rows 8 (q / 2) + j / 4 (+ 4, + 16) and outputs
//    16 (q % 2) + 4 (j % 4): the 8 rows of one read have 8 different f, so
//    its 64 lanes touch 32 distinct chunks.
// WGRAD contracts over a group's rows, any number of them: steps past the
// group's end load a zero line instead, and the step count is rounded up
// to even.
enum { BP_FPROP = 0, BP_DGRAD = 1, BP_WGRAD = 2 };

template <int TM>
struct Bp {
  static constexpr int TN = 256;
  static constexpr int SLOT = (TM + TN) * 64;
  static constexpr int NSLOT = 3;
  static constexpr int LDS = NSLOT * SLOT;
  static constexpr int CA = TM / 64, CB = TN / 64, OPS = CA + CB;
  static constexpr int FI = TM / 64, FJ = 4;
};

// 1 KB of zeros: the load source of contraction rows past a group's end.
__device__ uint4 g_bp_zero[64];

template <int TM>
struct BpSrc {
  const uint8_t *Ab, *Bb;                      // panel bases
  uint32_t oa[Bp<TM>::CA], ob[Bp<TM>::CB];     // per-lane offsets of step 0
  uint32_t sa, sb;                             // bytes per step
  uint32_t dst;                                // LDS address of slot 0, this wave
};

__device__ __forceinline__ int bp_swz(int row) { return (row & 3) | (((row >> 3) & 1) << 2); }

// Per-lane byte offset (within a step) of the chunks of a KL operand of
// `rows` valid rows and row stride `ld` bytes.
template <int C>
__device__ __forceinline__ void bp_offsets_kl(uint32_t (&o)[C], int rows, uint32_t ld) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int i = 0; i < C; ++i) {
    const int c = tid + 256 * i, r = c >> 2, k = (c & 3) ^ ((r >> 2) & 3);
    o[i] = (uint32_t)min(r, rows - 1) * ld + 16u * k;
  }
}

// ... of an ML operand with `cols` valid outputs (a multiple of 8) and
// contraction-row stride `ld` bytes.
template <int C>
__device__ __forceinline__ void bp_offsets_ml(uint32_t (&o)[C], int cols, uint32_t ld) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int i = 0; i < C; ++i) {
    const int c = tid + 256 * i, r = c >> 5, x = (c & 31) ^ (4 * bp_swz(r));
    o[i] = (uint32_t)r * ld + 16u * (uint32_t)min(x, cols / 8 - 1);
  }
}

// Request step kt into `slot`.  WGRAD: contraction rows at or past `len`
// read zeros.
template <int TM, int KIND>
__device__ __forceinline__ void bp_issue(const BpSrc<TM> &L, int kt, int slot, int len) {
  using C = Bp<TM>;
  const uint32_t base = L.dst + (uint32_t)slot * C::SLOT;
  const uint8_t *zero = reinterpret_cast<const uint8_t *>(g_bp_zero) + 16 * (threadIdx.x & 63);
  const int r0 = kt * 32 + ((int)threadIdx.x >> 5);  // contraction row of chunk 0 (ML)
#pragma unroll
  for (int i = 0; i < C::CA; ++i) {
    const uint8_t *src = L.Ab + (L.oa[i] + (uint32_t)kt * L.sa);
    if (KIND == BP_WGRAD && r0 + 8 * i >= len) src = zero;
    dma16(src, base + i * 4096);
  }
#pragma unroll
  for (int i = 0; i < C::CB; ++i) {
    const uint8_t *src = L.Bb + (L.ob[i] + (uint32_t)kt * L.sb);
    if (KIND == BP_WGRAD && r0 + 8 * i >= len) src = zero;
    dma16(src, base + TM * 64 + i * 4096);
  }
}

template <int TM>
struct BpFrags {
  uint4 a[Bp<TM>::FI][2], b[Bp<TM>::FJ][2];  // [fragment][16-K sub-step]
};

typedef short pqm_v4s __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) pqm_v4s pqm_lds_v4s;

__device__ __forceinline__ uint2 lds_read_tr16(const uint8_t *p) {
  const pqm_v4s v =
      __builtin_amdgcn_ds_read_tr16_b64_v4i16((pqm_lds_v4s *)(const_cast<uint8_t *>(p)));
  return __builtin_bit_cast(uint2, v);
}

// Fragments of one operand (F fragments of 32 outputs) from the ring region
// `reg`.  KL: off[0] / off[1] = the lane's chunk-h / chunk-(2+h) offsets of
// fragment 0, fragments 2048 bytes apart.  ML: off[f] = the lane's offset for
// fragment f; sub-step s, read r at + (16 s + 4 r) * 512.
template <bool ML>
__device__ __forceinline__ void bp_read_frag(const uint8_t *reg, const int *off, int f,
                                             uint4 (&fr)[2]) {
  if (ML) {
    const uint8_t *p = reg + off[f];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const uint2 r0 = lds_read_tr16(p + (16 * s) * 512);
      const uint2 r1 = lds_read_tr16(p + (16 * s + 4) * 512);
      fr[s] = make_uint4(r0.x, r0.y, r1.x, r1.y);
    }
  } else {
    fr[0] = *reinterpret_cast<const uint4 *>(reg + off[0] + 2048 * f);
    fr[1] = *reinterpret_cast<const uint4 *>(reg + off[1] + 2048 * f);
  }
}

template <int F, bool ML>
__device__ __forceinline__ void bp_read_op(const uint8_t *reg, const int *off, uint4 (&fr)[F][2]) {
#pragma unroll
  for (int f = 0; f < F; ++f) bp_read_frag<ML>(reg, off, f, fr[f]);
}

template <int KIND, int TM>
__device__ __forceinline__ void bp_read(const uint8_t *lds, int slot, const int *offA,
                                        const int *offB, BpFrags<TM> &F) {
  const uint8_t *reg = lds + slot * Bp<TM>::SLOT;
  bp_read_op<Bp<TM>::FI, KIND == BP_WGRAD>(reg, offA, F.a);
  bp_read_op<Bp<TM>::FJ, KIND != BP_FPROP>(reg, offB, F.b);
}

// Step kt from `slot` (operands in `cur`): as mx3_step.
template <int KIND, int TM>
__device__ __forceinline__ void bp_step(const BpSrc<TM> &L, const uint8_t *lds, const int *offA,
                                        const int *offB, int kt, int nk, int slot, int len,
                                        v16f (&acc)[Bp<TM>::FI][Bp<TM>::FJ],
                                        const BpFrags<TM> &cur, BpFrags<TM> &next) {
  using C = Bp<TM>;
  vm_wait<C::OPS>();
  lgkm_wait0();
  __builtin_amdgcn_s_barrier();
  // as mx3_step: after each MFMA a slice of the step's other work, two of
  // the refill loads of step kt+3 or one fragment's reads of step kt+1
  const int rk = min(kt + 3, nk - 1);
  const uint32_t base = L.dst + (uint32_t)slot * C::SLOT;
  const uint8_t *zero = reinterpret_cast<const uint8_t *>(g_bp_zero) + 16 * (threadIdx.x & 63);
  const int r0 = rk * 32 + ((int)threadIdx.x >> 5);  // contraction row of chunk 0 (ML)
  const uint8_t *reg = lds + (slot == 2 ? 0 : slot + 1) * C::SLOT;
  constexpr int NL = C::CA + C::CB, ND = (NL + 1) / 2, NM = 2 * C::FI * C::FJ;
  static_assert(NM - ND >= C::FI + C::FJ, "a slice for every fragment");
#pragma unroll
  for (int m = 0; m < NM; ++m) {
    const int sub = m / (C::FI * C::FJ), j = (m / C::FI) % C::FJ, i = m % C::FI;
    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(v8bf, cur.b[j][sub]),
                                                        __builtin_bit_cast(v8bf, cur.a[i][sub]),
                                                        acc[i][j], 0, 0, 0);
    if (m < ND) {
#pragma unroll
      for (int q = 2 * m; q < 2 * m + 2 && q < NL; ++q) {
        const bool isa = q < C::CA;
        const int ii = isa ? q : q - C::CA;
        const uint8_t *src = isa ? L.Ab + (L.oa[ii] + (uint32_t)rk * L.sa)
                                 : L.Bb + (L.ob[ii] + (uint32_t)rk * L.sb);
        if (KIND == BP_WGRAD && r0 + 8 * ii >= len) src = zero;
        dma16(src, base + (isa ? 0 : TM * 64) + ii * 4096);
      }
    } else if (m - ND < C::FI) {
      bp_read_frag<KIND == BP_WGRAD>(reg, offA, m - ND, next.a[m - ND]);
    } else if (m - ND - C::FI < C::FJ) {
      bp_read_frag<KIND != BP_FPROP>(reg, offB, m - ND - C::FI, next.b[m - ND - C::FI]);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

// One output tile.  Operand panels start at Ab / Bb (bytes); a_lim / b_lim
// are the valid rows (KL) or outputs (ML) of each; lda / ldb their row
// strides in bytes (KL: token / weight rows; ML: contraction rows).  len is
// the contraction length (WGRAD: the group's rows; otherwise K); the output
// rows row0 .. row_end-1, columns col0 .., row stride ldo.
struct BpArgs {
  const uint8_t *Ab, *Bb;
  int a_lim, b_lim;
  uint32_t lda, ldb;
  int len;
  void *out;
  int64_t ldo, row0, row_end, col0;
  const float *bias;  // FPROP: the expert's bias row, or null
};

template <int KIND, bool OUT_F32, int TM>
__device__ __forceinline__ void bp_tile(const BpArgs &p, uint8_t *lds) {
  static_assert(KIND != BP_WGRAD || TM == 256, "the ML layout is 256 outputs wide");
  using C = Bp<TM>;
  constexpr int FI = C::FI, FJ = C::FJ;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1, h = lane >> 5, r32 = lane & 31;
  BpSrc<TM> L;
  L.Ab = p.Ab;
  L.Bb = p.Bb;
  L.dst = __builtin_amdgcn_readfirstlane(lds_addr(lds) + (uint32_t)wave * 1024u);
  if (KIND == BP_WGRAD) {
    bp_offsets_ml<C::CA>(L.oa, p.a_lim, p.lda);
    L.sa = 32u * p.lda;
  } else {
    bp_offsets_kl<C::CA>(L.oa, p.a_lim, p.lda);
    L.sa = 64u;
  }
  if (KIND == BP_FPROP) {
    bp_offsets_kl<C::CB>(L.ob, p.b_lim, p.ldb);
    L.sb = 64u;
  } else {
    bp_offsets_ml<C::CB>(L.ob, p.b_lim, p.ldb);
    L.sb = 32u * p.ldb;
  }
  // lane 16 q + j of an ML read: rows 8 (q / 2) + j / 4 (+ 4 r + 16 s),
  // outputs 16 (q % 2) + 4 (j % 4) of the fragment; XOR of the row's swizzle
  const int q = lane >> 4, jj = lane & 15;
  const int rb0 = (8 * (q >> 1) + (jj >> 2)) * 512 + (2 * (q & 1) + ((jj >> 1) & 1)) * 16 +
                  8 * (jj & 1);
  const int xs = 64 * ((jj >> 2) | ((q >> 1) << 2));
  int offA[FI > 2 ? FI : 2], offB[FJ];
  if (KIND == BP_WGRAD) {
#pragma unroll
    for (int f = 0; f < FI; ++f) offA[f] = rb0 + ((2 * (wm * (TM / 2) + 32 * f)) ^ xs);
  } else {
    const int ra = wm * (TM / 2) + r32;
    offA[0] = mx3_off(ra, h);
    offA[1] = mx3_off(ra, 2 + h);
  }
  if (KIND == BP_FPROP) {
    const int rb = wn * 128 + r32;
    offB[0] = TM * 64 + mx3_off(rb, h);
    offB[1] = TM * 64 + mx3_off(rb, 2 + h);
  } else {
#pragma unroll
    for (int f = 0; f < FJ; ++f) offB[f] = TM * 64 + rb0 + ((2 * (wn * 128 + 32 * f)) ^ xs);
  }

  v16f acc[FI][FJ];
#pragma unroll
  for (int i = 0; i < FI; ++i)
#pragma unroll
    for (int j = 0; j < FJ; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  const int nk = 2 * ((p.len + 63) / 64);  // steps of 32, rounded up to even
  if (nk > 0) {
    bp_issue<TM, KIND>(L, 0, 0, p.len);
    bp_issue<TM, KIND>(L, 1, 1, p.len);
    bp_issue<TM, KIND>(L, min(2, nk - 1), 2, p.len);
    vm_wait<2 * C::OPS>();  // step 0
    __builtin_amdgcn_s_barrier();
    BpFrags<TM> F0, F1;
    bp_read<KIND, TM>(lds, 0, offA, offB, F0);
    int slot = 0;
    for (int kt = 0; kt < nk; kt += 2) {
      bp_step<KIND, TM>(L, lds, offA, offB, kt, nk, slot, p.len, acc, F0, F1);
      slot = slot == 2 ? 0 : slot + 1;
      bp_step<KIND, TM>(L, lds, offA, offB, kt + 1, nk, slot, p.len, acc, F1, F0);
      slot = slot == 2 ? 0 : slot + 1;
    }
    vm_wait<0>();  // no load may still target this workgroup's LDS at exit
  }
#pragma unroll
  for (int i = 0; i < FI; ++i)
#pragma unroll
    for (int j = 0; j < FJ; ++j)
      mx3_store<OUT_F32>(acc[i][j], p.out, p.ldo, p.row0, p.row_end, p.col0,
                         wm * (TM / 2) + 32 * i, wn * 128 + 32 * j, p.bias);
}

// FPROP / DGRAD: row tiles of 256 tokens over the groups (an expert's last
// tile of <= 128 rows as 128 x 256), 256 output columns; K % 64 == 0.
// WGRAD: tile (g, 256 rows n, 256 columns k) of Y_g, contraction over the
// group's rows.
template <int KIND, bool OUT_F32, bool BIAS = false>
__global__ __launch_bounds__(256, 1) void k_gemm_bf16_pipe(
    const uint16_t *__restrict__ A, const uint16_t *__restrict__ B,
    const int64_t *__restrict__ offsets, int64_t G, int64_t N, int64_t K, int64_t ntn,
    int64_t ntk, void *__restrict__ out, const float *__restrict__ bias) {
  static_assert(Bp<128>::LDS <= Bp<256>::LDS, "LDS of the half tile");
  __shared__ __attribute__((aligned(16))) uint8_t lds[Bp<256>::LDS];
  __shared__ int64_t sh[4];
  BpArgs p;
  p.bias = nullptr;
  if constexpr (KIND == BP_WGRAD) {
    const int64_t t = blockIdx.x;
    const int64_t g = t / (ntn * ntk);
    const int64_t n0 = ((t / ntk) % ntn) * 256, k0 = (t % ntk) * 256;
    const int64_t m0 = offsets[g], m1 = offsets[g + 1];
    p.Ab = reinterpret_cast<const uint8_t *>(A + m0 * N + n0);
    p.Bb = reinterpret_cast<const uint8_t *>(B + m0 * K + k0);
    p.a_lim = (int)min(N - n0, (int64_t)256);
    p.b_lim = (int)min(K - k0, (int64_t)256);
    p.lda = (uint32_t)(N * 2);
    p.ldb = (uint32_t)(K * 2);
    p.len = (int)(m1 - m0);
    p.out = OUT_F32 ? (void *)(static_cast<float *>(out) + g * N * K)
                    : (void *)(static_cast<uint16_t *>(out) + g * N * K);
    p.ldo = K;
    p.row0 = n0;
    p.row_end = N;
    p.col0 = k0;
    bp_tile<KIND, OUT_F32, 256>(p, lds);
  } else {
  TileInfo ti;
  if (!lookup_row_tile<256, 256>(offsets, G, ntn, ti, sh)) return;
  p.Ab = reinterpret_cast<const uint8_t *>(A + ti.row0 * K);
  p.a_lim = (int)min(ti.row_end - ti.row0, (int64_t)256);
  p.lda = (uint32_t)(K * 2);
  if (KIND == BP_FPROP) {
    p.Bb = reinterpret_cast<const uint8_t *>(B + (ti.g * N + ti.n0) * K);
    p.ldb = (uint32_t)(K * 2);
  } else {
    p.Bb = reinterpret_cast<const uint8_t *>(B + ti.g * K * N + ti.n0);
    p.ldb = (uint32_t)(N * 2);
  }
  p.b_lim = (int)min(N - ti.n0, (int64_t)256);
  p.len = (int)K;
  p.out = out;
  p.ldo = N;
  p.row0 = ti.row0;
  p.row_end = ti.row_end;
  p.col0 = ti.n0;
  if (KIND == BP_FPROP && BIAS) p.bias = bias + ti.g * N;
  if (ti.row_end - ti.row0 <= 128)
    bp_tile<KIND, OUT_F32, 128>(p, lds);
  else
    bp_tile<KIND, OUT_F32, 256>(p, lds);
  }
}

// ------------------------------------------------------------------ NVFP4
//
// E2M1 x E4M3 (q * s_b) has at most 2 + 4 significant bits and lies in
// [2^-10, 2688], so it is exact in fp16; the matrix cores then see the exact
// block-scaled operand values, and the FP32 outer scales (per token for A,
// per expert tensor for B) multiply the binary32 accumulator.  Per-16 E4M3
// scales are not a CDNA4 matrix-core scale format, hence the decode while
// staging into LDS.
//
// Decode of one 32-bit word (8 nibbles, element 2j in the low nibble of
// byte j): the magnitude codes are looked up as the high byte of the fp16
// value in an 8-entry byte table with v_perm_b32 (four lookups per
// instruction), the sign bit is ORed in, the bytes are interleaved into
// fp16 pairs and multiplied by s_b with one packed fp16 multiply per pair.

typedef _Float16 pqm_v2h __attribute__((ext_vector_type(2)));

__device__ __forceinline__ void nvfp4_word_to_f16(uint32_t w, pqm_v2h sb2, uint32_t out[4]) {
  const uint32_t LUT_LO = 0x3E3C3800u, LUT_HI = 0x46444240u;  // 0,.5,1,1.5 | 2,3,4,6
  const uint32_t hlo = __builtin_amdgcn_perm(LUT_HI, LUT_LO, w & 0x07070707u) |
                       ((w & 0x08080808u) << 4);  // elements 0,2,4,6
  const uint32_t hhi = __builtin_amdgcn_perm(LUT_HI, LUT_LO, (w >> 4) & 0x07070707u) |
                       (w & 0x80808080u);         // elements 1,3,5,7
  const uint32_t sel[4] = {0x040C000Cu, 0x050C010Cu, 0x060C020Cu, 0x070C030Cu};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t pr = __builtin_amdgcn_perm(hhi, hlo, sel[j]);
    const pqm_v2h v = __builtin_bit_cast(pqm_v2h, pr) * sb2;  // exact
    out[j] = __builtin_bit_cast(uint32_t, v);
  }
}

// Stage a 128-row x 64-element NVFP4 operand tile as fp16 [row][k] in LDS.
// Lane t owns row t/2, elements 32 (t%2) .. +31 of the step: 16 bytes of
// packed data and 2 scale bytes.
struct Nvfp4Loader {
  uint4 v;
  uint32_t sc;  // two E4M3 bytes
  __device__ void load(const uint8_t *__restrict__ q, const uint8_t *__restrict__ s,
                       int64_t rows, int64_t k0, int64_t K) {
    const int r = threadIdx.x >> 1, h = threadIdx.x & 1;
    const int64_t e = k0 + 32 * h;
    v = make_uint4(0, 0, 0, 0);
    sc = 0;
    if (r < rows && e < K) {
      const uint8_t *qr = q + r * (K / 2) + e / 2;
      if (e + 32 <= K) {
        v = *reinterpret_cast<const uint4 *>(qr);
        sc = (uint32_t)s[r * (K / 16) + e / 16] | ((uint32_t)s[r * (K / 16) + e / 16 + 1] << 8);
      } else {  // K % 16 == 0: a 16-element remainder
        const uint2 u = *reinterpret_cast<const uint2 *>(qr);
        v.x = u.x;
        v.y = u.y;
        sc = (uint32_t)s[r * (K / 16) + e / 16];
      }
    }
  }
  __device__ void store(uint8_t *lds) const {
    const int r = threadIdx.x >> 1, h = threadIdx.x & 1;
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    uint32_t o[16];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const _Float16 sbh = (_Float16)e4m3_value((sc >> (8 * (i >> 1))) & 0x7Fu);
      const pqm_v2h sb2 = {sbh, sbh};
      nvfp4_word_to_f16(w[i], sb2, o + 4 * i);
    }
    uint4 *dst = reinterpret_cast<uint4 *>(lds + r * GT_PITCH + 64 * h);
#pragma unroll
    for (int i = 0; i < 4; ++i) dst[i] = make_uint4(o[4 * i], o[4 * i + 1], o[4 * i + 2], o[4 * i + 3]);
  }
};

__device__ __forceinline__ v8h frag_f16(const uint8_t *lds, int row, int s) {
  const int lane = threadIdx.x & 63;
  const uint4 v = *reinterpret_cast<const uint4 *>(lds + row * GT_PITCH + 32 * s +
                                                   16 * (lane >> 5));
  return __builtin_bit_cast(v8h, v);
}

template <bool OUT_F32>
__global__ __launch_bounds__(256) void k_gemm_nvfp4(
    const uint8_t *__restrict__ A, const uint8_t *__restrict__ As,
    const float *__restrict__ Ao, const uint8_t *__restrict__ B,
    const uint8_t *__restrict__ Bs, const float *__restrict__ Bo, int64_t b_rps,
    const int64_t *__restrict__ offsets, int64_t G, int64_t N, int64_t K, int64_t ntn,
    void *__restrict__ out, const float *__restrict__ bias) {
  __shared__ __attribute__((aligned(16))) uint8_t lA[GT_M * GT_PITCH];
  __shared__ __attribute__((aligned(16))) uint8_t lB[GT_N * GT_PITCH];
  __shared__ int64_t sh[4];
  TileInfo ti;
  if (!lookup_row_tile(offsets, G, ntn, ti, sh)) return;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int64_t rows_a = ti.row_end - ti.row0;
  const int64_t rows_b = N - ti.n0;
  const uint8_t *Aq = A + ti.row0 * (K / 2), *Asb = As + ti.row0 * (K / 16);
  const uint8_t *Bq = B + (ti.g * N + ti.n0) * (K / 2), *Bsb = Bs + (ti.g * N + ti.n0) * (K / 16);
  v16f acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
  Nvfp4Loader la, lb;
  la.load(Aq, Asb, rows_a, 0, K);
  lb.load(Bq, Bsb, rows_b, 0, K);
  const int nk = (int)((K + 63) / 64);
  for (int kt = 0; kt < nk; ++kt) {
    la.store(lA);
    lb.store(lB);
    __syncthreads();
    if (kt + 1 < nk) {
      la.load(Aq, Asb, rows_a, (int64_t)(kt + 1) * 64, K);
      lb.load(Bq, Bsb, rows_b, (int64_t)(kt + 1) * 64, K);
    }
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      v8h fa[2], fb[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        fa[i] = frag_f16(lA, wm * 64 + 32 * i + (lane & 31), s);
        fb[i] = frag_f16(lB, wn * 64 + 32 * i + (lane & 31), s);
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(fa[i], fb[j], acc[i][j], 0, 0, 0);
    }
    __syncthreads();
  }
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int64_t col = ti.n0 + wn * 64 + 32 * j + (lane & 31);
    const float ab = col < N ? Bo[(ti.g * N + col) / b_rps] : 0.0f;
#pragma unroll
    for (int i = 0; i < 2; ++i)
      store_acc<OUT_F32>(acc[i][j], out, N, ti.row0, ti.row_end, ti.n0, N, wm * 64 + 32 * i,
                         wn * 64 + 32 * j, Ao, ab, bias ? bias + ti.g * N : nullptr);
  }
}

// --------------------------------------------- NVFP4, pipelined large tiles
//
// The same ring and tiles as the MXFP8 / BF16 pipelines, carrying the packed
// operands: a step is 128 K, i.e. 64 bytes of E2M1 and 8 E4M3 block scales
// per row, both loaded straight into LDS (slot: A data, B data, A scales,
// B scales).  The fp16 operand values are produced while the fragments are
// read: lane half h takes bytes 32 h .. 32 h + 31 of each row (two 16-byte
// reads) and the 4 scale bytes of the blocks they cover (one 4-byte read);
// sub-step s (0..7) contracts the 8 elements 64 h + 8 s .. of each lane (the
// same K permutation for both operands, and each group of 8 lies in one
// 16-element block).  A block scale s_b = M 2^E (M in [1, 2), 4 significant
// bits) is applied in two exact steps: the scaled FP4 -> f16 pair conversion
// (v_cvt_scalef32_pk_f16_fp4, which scales by the power of two 2^E; checked
// exhaustively on gfx950) and one packed f16 multiply by M; q s_b has at most
// 6 significant bits in [2^-10, 2688], exact in f16.  The outer scales
// multiply the binary32 accumulator in the epilogue as in k_gemm_nvfp4.
// Tile configuration: TMR_ rows of A and TN_ rows of B (output columns) in
// a slot; WM_ waves along M: 2 gives 2 x 2 waves of (TMR/2) x (TN/2)
// outputs, 1 gives 1 x 4 waves of (32 FI_) x (TN/4) outputs, FI_ A fragments
// per wave (rows of the slot past 32 FI_ WM_ are loaded but not multiplied,
// so an expert's last tile of few rows multiplies only whole 32-row groups).
// With 1 x 4 waves every wave decodes the tile's A fragments and its own
// quarter of B: 8 decodes per 16 MFMAs at 128 x 512 against 10 with 2 x 2.
// AQ: the ring loads the A operand's codes and block scales from memory;
// otherwise the workgroup writes them into each slot itself (the FC2 kernel
// with online amax) and the ring carries B only.
template <int TMR_, int TN_, int WM_, int FI_, bool AQ_ = true>
struct Np {
  static constexpr int TMR = TMR_, TN = TN_, WM = WM_, ROWS = TMR + TN;
  static constexpr bool AQ = AQ_;
  static constexpr int SC = ROWS * 64;        // scale area offset in a slot
  static constexpr int SLOT = ROWS * 72;
  static constexpr int NSLOT = 3;  // 4 slots measured no faster
  static constexpr int LDS = NSLOT * SLOT;
  static constexpr int CA = TMR / 64, CB = TN / 64;  // 16-byte data chunks per lane
  static constexpr int NS = ROWS / 128;              // 4-byte scale loads per lane
  static constexpr int CAL = AQ ? CA : 0;            // A chunks the ring loads
  static constexpr int NS0 = AQ ? 0 : TMR / 128;     // first scale load of the ring (A rows first)
  static constexpr int OPS = CAL + CB + NS - NS0;    // ring loads per lane per step
  static_assert(AQ || TMR % 128 == 0, "A scale rows are whole scale loads");
  static constexpr int FI = FI_, FJ = TN * WM / 128;
  static constexpr int WROWS = TMR / WM, WCOLS = TN * WM / 4;  // a wave's row / column offset step
  static_assert(FI * 32 <= WROWS && FJ * 32 == WCOLS, "wave tile");
};
using NpPipe256 = Np<256, 256, 2, 4>;
using NpPipe128 = Np<128, 256, 2, 2>;

// The ring's load sources (the same type for every fragment count of a tile
// shape, so a persistent loop can keep one across tiles).
template <int CA, int CB, int NS>
struct NpRing {
  const uint8_t *Ab, *Bb, *Asb, *Bsb;
  uint32_t oa[CA], ob[CB], os[NS];  // step-0 offsets
  uint32_t dst, sdst;  // LDS addresses of slot 0's data and scales, this wave
};
template <class C>
using NpSrc = NpRing<C::CA, C::CB, C::NS>;

// Point the ring's loads at the tile (g, rows row0 .. row_end - 1, columns
// n0 ..): per-lane offsets of step 0 (rows past the tile's end clamped to its
// last row).
template <class C>
__device__ __forceinline__ void np_loader(NpSrc<C> &L, const uint8_t *__restrict__ A,
                                          const uint8_t *__restrict__ As,
                                          const uint8_t *__restrict__ B,
                                          const uint8_t *__restrict__ Bs, int64_t N, int64_t K,
                                          int64_t g, int64_t row0, int64_t row_end, int64_t n0) {
  int tid = threadIdx.x;
  asm volatile("" : "+v"(tid));  // recomputed where called, not kept live across a loop
  const uint32_t KD = (uint32_t)(K / 2), KS = (uint32_t)(K / 16);  // row bytes of data / scales
  const int rows_a = (int)min(row_end - row0, (int64_t)C::TMR);
  const int rows_b = (int)min(N - n0, (int64_t)C::TN);
  L.Ab = A + row0 * (int64_t)KD;
  L.Bb = B + (g * N + n0) * (int64_t)KD;
  L.Asb = As + row0 * (int64_t)KS;
  L.Bsb = Bs + (g * N + n0) * (int64_t)KS;
#pragma unroll
  for (int i = 0; i < C::CA; ++i) {
    const int c = tid + 256 * i, r = c >> 2, k = (c & 3) ^ ((r >> 2) & 3);
    L.oa[i] = (uint32_t)min(r, rows_a - 1) * KD + 16u * k;
  }
#pragma unroll
  for (int i = 0; i < C::CB; ++i) {
    const int c = tid + 256 * i, r = c >> 2, k = (c & 3) ^ ((r >> 2) & 3);
    L.ob[i] = (uint32_t)min(r, rows_b - 1) * KD + 16u * k;
  }
#pragma unroll
  for (int i = 0; i < C::NS; ++i) {
    const int d = tid + 256 * i, r = d >> 1, half = d & 1;
    L.os[i] = r < C::TMR ? (uint32_t)min(r, rows_a - 1) * KS + 4u * half
                          : (uint32_t)min(r - C::TMR, rows_b - 1) * KS + 4u * half;
  }
}

// Loads q0 .. q1-1 of a step's ring loads: A chunks (when the ring carries
// A), B chunks, then scale words (dwords 256 i + tid: rows 128 i .., A rows
// first).
template <class C, int Q0, int Q1>
__device__ __forceinline__ void np_issue_range(const NpSrc<C> &L, int kt, int slot) {
  static_assert(0 <= Q0 && Q0 <= Q1 && Q1 <= C::OPS, "load range within the step's loads");
  const uint32_t kb = (uint32_t)kt * 64u, ks = (uint32_t)kt * 8u;
  const uint32_t base = L.dst + (uint32_t)slot * C::SLOT, sbase = L.sdst + (uint32_t)slot * C::SLOT;
#pragma unroll
  for (int q = Q0; q < Q1; ++q) {
    if (q < C::CAL) {
      dma16(L.Ab + (L.oa[q] + kb), base + q * 4096);
    } else if (q < C::CAL + C::CB) {
      dma16(L.Bb + (L.ob[q - C::CAL] + kb), base + C::TMR * 64 + (q - C::CAL) * 4096);
    } else {
      const int i = q - C::CAL - C::CB + C::NS0;
      dma4((128 * i < C::TMR ? L.Asb : L.Bsb) + (L.os[i] + ks), sbase + i * 1024);
    }
  }
}

// Step kt into slot `slot`: all of its ring loads.
template <class C>
__device__ __forceinline__ void np_issue(const NpSrc<C> &L, int kt, int slot) {
  np_issue_range<C, 0, C::OPS>(L, kt, slot);
}

// Start of the k-th of 8 near-equal ranges of a step's C::OPS loads (k = 8:
// the end); ranges past the last load are empty.
template <class C>
__host__ __device__ constexpr int np_cut(int k) {
  return k * ((C::OPS + 7) / 8) < C::OPS ? k * ((C::OPS + 7) / 8) : C::OPS;
}

struct NpLane {
  int a0, a1, b0, b1;  // chunk offsets (2h, 2h+1) of the first A / B row
  int sa, sb;          // scale-word offsets of the first A / B row
};

// A lane's raw operands of one step, per fragment 32 bytes in two halves:
// half 0 (chunk 2h: words 0..3 = sub-steps 0..3 = blocks 0, 1) and half 1
// (chunk 2h + 1: sub-steps 4..7 = blocks 2, 3), plus one word holding the
// 4 scale bytes of the lane's blocks.
template <class C>
struct NpHalf {
  uint4 a[C::FI], b[C::FJ];
};
template <class C>
struct NpWords {
  uint32_t a[C::FI], b[C::FJ];
};

template <class C, int HALF>
__device__ __forceinline__ void np_read_half(const uint8_t *lds, int slot, const NpLane &o,
                                             NpHalf<C> &R) {
  const uint8_t *cur = lds + slot * C::SLOT;
#pragma unroll
  for (int i = 0; i < C::FI; ++i)
    R.a[i] = *reinterpret_cast<const uint4 *>(cur + (HALF ? o.a1 : o.a0) + 2048 * i);
#pragma unroll
  for (int j = 0; j < C::FJ; ++j)
    R.b[j] = *reinterpret_cast<const uint4 *>(cur + (HALF ? o.b1 : o.b0) + 2048 * j);
}

template <class C>
__device__ __forceinline__ void np_read_words(const uint8_t *lds, int slot, const NpLane &o,
                                              NpWords<C> &W) {
  const uint8_t *cur = lds + slot * C::SLOT;
#pragma unroll
  for (int i = 0; i < C::FI; ++i) W.a[i] = *reinterpret_cast<const uint32_t *>(cur + o.sa + 256 * i);
#pragma unroll
  for (int j = 0; j < C::FJ; ++j) W.b[j] = *reinterpret_cast<const uint32_t *>(cur + o.sb + 256 * j);
}

// Block scale byte `byte` (0..3) of `sw` as 2^E (binary32) and M (f16 pair).
struct NpScale {
  float p2;
  uint32_t m2;
};

template <int BYTE>
__device__ __forceinline__ NpScale np_scale(uint32_t sw) {
  // E4M3 -> binary32 exactly (every E4M3 value is a normal binary32)
  const uint32_t f = __float_as_uint(__builtin_amdgcn_cvt_f32_fp8((int)sw, BYTE));
  NpScale r;
  r.p2 = __uint_as_float(f & 0x7F800000u);
  const uint32_t m16 = ((f >> 13) & 0x380u) | 0x3C00u;  // 1.mmm in f16
  r.m2 = m16 | (m16 << 16);
  return r;
}

// 8 fp16 operand values of word w (sub-step) under block scale sc.
__device__ __forceinline__ v8h np_decode(uint32_t w, const NpScale &sc) {
  const pqm_v2h m = __builtin_bit_cast(pqm_v2h, sc.m2);
  const pqm_v2h x0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, sc.p2, 0) * m;
  const pqm_v2h x1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, sc.p2, 1) * m;
  const pqm_v2h x2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, sc.p2, 2) * m;
  const pqm_v2h x3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, sc.p2, 3) * m;
  return v8h{x0[0], x0[1], x1[0], x1[1], x2[0], x2[1], x3[0], x3[1]};
}

template <int WORD>
__device__ __forceinline__ uint32_t u4_word(const uint4 &u) {
  return WORD == 0 ? u.x : (WORD == 1 ? u.y : (WORD == 2 ? u.z : u.w));
}

// Block scales of one block of every fragment, and the fp16 operands of one
// sub-step.
template <class C>
struct NpScales {
  NpScale a[C::FI], b[C::FJ];
};
template <class C>
struct NpDec {
  v8h a[C::FI], b[C::FJ];
};

template <class C, int BLK>
__device__ __forceinline__ void np_scales(const NpWords<C> &W, NpScales<C> &S) {
#pragma unroll
  for (int i = 0; i < C::FI; ++i) S.a[i] = np_scale<BLK>(W.a[i]);
#pragma unroll
  for (int j = 0; j < C::FJ; ++j) S.b[j] = np_scale<BLK>(W.b[j]);
}

template <class C, int WORD>
__device__ __forceinline__ void np_dec(const NpHalf<C> &R, const NpScales<C> &S, NpDec<C> &X) {
#pragma unroll
  for (int i = 0; i < C::FI; ++i) X.a[i] = np_decode(u4_word<WORD>(R.a[i]), S.a[i]);
#pragma unroll
  for (int j = 0; j < C::FJ; ++j) X.b[j] = np_decode(u4_word<WORD>(R.b[j]), S.b[j]);
}

// The MFMAs of one decoded sub-step; the instructions placed before them in
// the same scheduling region (the next sub-step's decode) are spread between
// them: each MFMA keeps the matrix core busy for 32 cycles while the wave
// issues up to 6 VALU instructions.
template <class C>
__device__ __forceinline__ void np_mfmas(const NpDec<C> &X,
                                         v16f (&acc)[C::FI][C::FJ]) {
#pragma unroll
  for (int j = 0; j < C::FJ; ++j)
#pragma unroll
    for (int i = 0; i < C::FI; ++i)
      acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(X.b[j], X.a[i], acc[i][j], 0, 0, 0);
#pragma unroll
  for (int m = 0; m < C::FI * C::FJ; ++m) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
    __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);  // then VALU
  }
  __builtin_amdgcn_sched_barrier(0);
}

// One 128-K step, software-pipelined over its 8 sub-steps.  On entry R0 / R1
// hold this step's raw halves, W its scale words and X its decoded sub-step
// 0.  Sub-step s + 1 is decoded while the MFMAs of s run.  Once sub-step 3
// is decoded (half 0 dead) half 0 and the scale words of step kt + 1 are
// read from slot `nslot` into R0 / W; once sub-step 7 is, half 1 into R1;
// and the last sub-step's MFMAs cover the decode of step kt + 1's sub-step
// 0.  So one set of raw registers serves two steps, and the registers saved
// hold the second decoded sub-step.
template <class C>
__device__ __forceinline__ void np_step(const NpSrc<C> &L, int rk, int slot,
                                        const uint8_t *lds, const NpLane &o, int nslot,
                                        v16f (&acc)[C::FI][C::FJ], NpHalf<C> &R0,
                                        NpHalf<C> &R1, NpWords<C> &W, NpScales<C> &S,
                                        NpDec<C> &X, NpDec<C> &Y) {
  // the refill of `slot` with step rk: load range k (np_cut) after the
  // MFMAs of sub-step k
  np_dec<C, 1>(R0, S, Y);                 // s = 1 (block 0)
  np_mfmas<C>(X, acc);                    // s = 0
  np_issue_range<C, np_cut<C>(0), np_cut<C>(1)>(L, rk, slot);
  np_scales<C, 1>(W, S);
  np_dec<C, 2>(R0, S, X);                 // s = 2 (block 1)
  np_mfmas<C>(Y, acc);                    // s = 1
  np_issue_range<C, np_cut<C>(1), np_cut<C>(2)>(L, rk, slot);
  np_dec<C, 3>(R0, S, Y);                 // s = 3
  np_mfmas<C>(X, acc);                    // s = 2
  np_issue_range<C, np_cut<C>(2), np_cut<C>(3)>(L, rk, slot);
  np_scales<C, 2>(W, S);
  np_dec<C, 0>(R1, S, X);                 // s = 4 (block 2)
  np_mfmas<C>(Y, acc);                    // s = 3
  np_issue_range<C, np_cut<C>(3), np_cut<C>(4)>(L, rk, slot);
  np_read_half<C, 0>(lds, nslot, o, R0);  // step kt + 1, half 0
  NpWords<C> Wn;
  np_read_words<C>(lds, nslot, o, Wn);
  __builtin_amdgcn_sched_barrier(0);
  np_dec<C, 1>(R1, S, Y);                 // s = 5
  np_mfmas<C>(X, acc);                    // s = 4
  np_issue_range<C, np_cut<C>(4), np_cut<C>(5)>(L, rk, slot);
  np_scales<C, 3>(W, S);
  np_dec<C, 2>(R1, S, X);                 // s = 6 (block 3)
  np_mfmas<C>(Y, acc);                    // s = 5
  np_issue_range<C, np_cut<C>(5), np_cut<C>(6)>(L, rk, slot);
  np_dec<C, 3>(R1, S, Y);                 // s = 7
  np_mfmas<C>(X, acc);                    // s = 6
  np_issue_range<C, np_cut<C>(6), np_cut<C>(7)>(L, rk, slot);
  np_read_half<C, 1>(lds, nslot, o, R1);  // step kt + 1, half 1
  __builtin_amdgcn_sched_barrier(0);
  W = Wn;
  np_scales<C, 0>(W, S);
  np_dec<C, 0>(R0, S, X);                 // step kt + 1, s = 0
  np_mfmas<C>(Y, acc);                    // s = 7
  np_issue_range<C, np_cut<C>(7), np_cut<C>(8)>(L, rk, slot);
}

// Store one transposed accumulator with the outer scales: as mx3_store, each
// value times alpha_a[row] * alpha_b(column) (the product exact in
// binary64, one rounding to binary32, then to bf16 for bf16 output).
// ab: the tile's column scales in LDS.  ROW_LOCAL: Ao holds the tile's row
// scales, indexed by the row within the tile (in LDS).  bias: the expert's
// bias row (binary32), added in binary64 before the one rounding, or null.
template <bool OUT_F32, bool ROW_LOCAL = false>
__device__ __forceinline__ void np_store(const v16f &acc, void *out, int64_t N, int64_t row0,
                                         int64_t row_end, int64_t n0, int rbase, int cbase,
                                         const float *__restrict__ Ao, const float *ab,
                                         const float *bias = nullptr) {
  const int lane = threadIdx.x & 63, h = lane >> 5;
  const int64_t row = row0 + rbase + (lane & 31);
  const double aa =
      row < row_end ? (double)(ROW_LOCAL ? Ao[rbase + (lane & 31)] : Ao[row]) : 0.0;
  const bool vec = (N & 7) == 0;
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    float lo[4], hi[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float a = acc[8 * p + e], b = acc[8 * p + 4 + e];
      const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(h ? a : b),
                                                       __float_as_uint(h ? a : b), false, false);
      const float got = __uint_as_float(h ? sw[0] : sw[1]);
      lo[e] = h ? got : a;
      hi[e] = h ? b : got;
    }
    const int c0 = cbase + 16 * p + 8 * h;  // column within the tile
    const int64_t col = n0 + c0;
    if (row >= row_end) continue;
    float v[8] = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    if (bias) {
#pragma unroll
      for (int e = 0; e < 8; ++e)
        v[e] = (float)((double)v[e] * (aa * (double)ab[c0 + e]) +
                       (double)bias[min(col + e, N - 1)]);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = (float)((double)v[e] * (aa * (double)ab[c0 + e]));
    }
    if (vec && col + 7 < N) {
      if (OUT_F32) {
        float *dst = static_cast<float *>(out) + row * N + col;
        *reinterpret_cast<float4 *>(dst) = make_float4(v[0], v[1], v[2], v[3]);
        *reinterpret_cast<float4 *>(dst + 4) = make_float4(v[4], v[5], v[6], v[7]);
      } else {
        const uint4 w = make_uint4(pk_bf16_rne(v[0], v[1]), pk_bf16_rne(v[2], v[3]),
                                   pk_bf16_rne(v[4], v[5]), pk_bf16_rne(v[6], v[7]));
        *reinterpret_cast<uint4 *>(static_cast<uint16_t *>(out) + row * N + col) = w;
      }
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        if (col + e < N) {
          if (OUT_F32)
            static_cast<float *>(out)[row * N + col + e] = v[e];
          else
            static_cast<uint16_t *>(out)[row * N + col + e] = (uint16_t)f32_to_bf16_rne(v[e]);
        }
      }
    }
  }
}

template <class C>
__device__ __forceinline__ void npo_rescale(const float *ratio, int wm, int r32,
                                            v16f (&acc)[C::FI][C::FJ]);

// One tile of the NVFP4 grouped GEMM.  With a ratio array (binary32
// [rows, K / 128], row-major from the tile's first row), each step first
// moves the accumulator rows by their ratio for that step, as the online-amax
// FC2 does (O = O (gs_prev / gs) + dO); rl: LDS for the tile's ratios,
// stored step-major (C::TMR per step).
template <bool OUT_F32, class C>
__device__ __forceinline__ void np_tile(const uint8_t *__restrict__ A,
                                        const uint8_t *__restrict__ As,
                                        const float *__restrict__ Ao,
                                        const uint8_t *__restrict__ B,
                                        const uint8_t *__restrict__ Bs, int64_t N, int64_t K,
                                        const TileInfo &ti, uint8_t *lds, const float *ab,
                                        void *__restrict__ out, const float *bias,
                                        const float *__restrict__ ratio = nullptr,
                                        float *rl = nullptr) {
  constexpr int FI = C::FI, FJ = C::FJ;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = C::WM == 2 ? wave >> 1 : 0, wn = C::WM == 2 ? wave & 1 : wave;
  const int h = lane >> 5, r32 = lane & 31;
  if (ratio) {  // before any ring load, so that the ring's load counts stay as they are
    const int nk = (int)(K / 128), rows = (int)min(ti.row_end - ti.row0, (int64_t)C::TMR);
    for (int i = tid; i < nk * C::TMR; i += 256) {
      const int kt = i / C::TMR, r = min(i % C::TMR, rows - 1);
      rl[i] = ratio[(ti.row0 + r) * nk + kt];
    }
    __syncthreads();
  }
  NpSrc<C> L;
  np_loader<C>(L, A, As, B, Bs, N, K, ti.g, ti.row0, ti.row_end, ti.n0);
  L.dst = __builtin_amdgcn_readfirstlane(lds_addr(lds) + (uint32_t)wave * 1024u);
  L.sdst = __builtin_amdgcn_readfirstlane(lds_addr(lds) + C::SC + (uint32_t)wave * 256u);
  NpLane o;
  {
    const int ra = wm * C::WROWS + r32, rb = wn * C::WCOLS + r32;
    o.a0 = mx3_off(ra, 2 * h);
    o.a1 = mx3_off(ra, 2 * h + 1);
    o.b0 = C::TMR * 64 + mx3_off(rb, 2 * h);
    o.b1 = C::TMR * 64 + mx3_off(rb, 2 * h + 1);
    o.sa = C::SC + ra * 8 + 4 * h;
    o.sb = C::SC + (C::TMR + rb) * 8 + 4 * h;
  }
  v16f acc[FI][FJ];
#pragma unroll
  for (int i = 0; i < FI; ++i)
#pragma unroll
    for (int j = 0; j < FJ; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  const int nk = (int)(K / 128);  // even, >= 2
#pragma unroll
  for (int s = 0; s < C::NSLOT; ++s) np_issue<C>(L, min(s, nk - 1), s);
  vm_wait<(C::NSLOT - 1) * C::OPS>();  // step 0
  __builtin_amdgcn_s_barrier();
  NpHalf<C> R0, R1;
  NpWords<C> W;
  NpScales<C> S;
  NpDec<C> X, Y;
  np_read_half<C, 0>(lds, 0, o, R0);
  np_read_half<C, 1>(lds, 0, o, R1);
  np_read_words<C>(lds, 0, o, W);
  np_scales<C, 0>(W, S);
  np_dec<C, 0>(R0, S, X);
  int slot = 0;
  for (int kt = 0; kt < nk; ++kt) {
    // own loads of step kt + 1 done (step kt + 2 may be pending), own reads
    // of slot kt % 3 (issued during step kt - 1) done; after the barrier
    // every wave's are, so step kt + 3 may refill the slot and step kt + 1
    // may be read
    vm_wait<C::OPS>();
    lgkm_wait0();
    __builtin_amdgcn_s_barrier();
    const int nslot = slot == C::NSLOT - 1 ? 0 : slot + 1;
    if (ratio) npo_rescale<C>(rl + kt * C::TMR, wm, r32, acc);
    // past the last step the reads take the slot's repeated last step (in
    // bounds; decoded, never multiplied)
    np_step<C>(L, min(kt + C::NSLOT, nk - 1), slot, lds, o, nslot, acc, R0, R1, W, S, X, Y);
    slot = nslot;
  }
  vm_wait<0>();
#pragma unroll
  for (int i = 0; i < FI; ++i)
#pragma unroll
    for (int j = 0; j < FJ; ++j)
      np_store<OUT_F32>(acc[i][j], out, N, ti.row0, ti.row_end, ti.n0, wm * C::WROWS + 32 * i,
                        wn * C::WCOLS + 32 * j, Ao, ab, bias);
}

// 256 x 256 tiles (an expert's last tile of <= 128 rows as 128 x 256);
// K % 256 == 0.
template <bool OUT_F32, bool BIAS>
__global__ __launch_bounds__(256, 1) void k_gemm_nvfp4_pipe(
    const uint8_t *__restrict__ A, const uint8_t *__restrict__ As,
    const float *__restrict__ Ao, const uint8_t *__restrict__ B,
    const uint8_t *__restrict__ Bs, const float *__restrict__ Bo, int64_t b_rps,
    const int64_t *__restrict__ offsets, int64_t G, int64_t N, int64_t K, int64_t ntn,
    void *__restrict__ out, const float *__restrict__ bias) {
  static_assert(NpPipe128::LDS <= NpPipe256::LDS, "LDS of the half tile");
  __shared__ __attribute__((aligned(16))) uint8_t lds[NpPipe256::LDS];
  __shared__ float ab[256];
  __shared__ int64_t sh[4];
  TileInfo ti;
  if (!lookup_row_tile<256, 256>(offsets, G, ntn, ti, sh)) return;
  {  // the tile's column scales alpha_b(n) = Bo[(g N + n) / b_rps]
    const int64_t col = ti.n0 + threadIdx.x;
    ab[threadIdx.x] = col < N ? Bo[(ti.g * N + col) / b_rps] : 0.0f;
  }
  __syncthreads();
  const float *bg = BIAS ? bias + ti.g * N : nullptr;
  if (ti.row_end - ti.row0 <= 128)
    np_tile<OUT_F32, NpPipe128>(A, As, Ao, B, Bs, N, K, ti, lds, ab, out, bg);
  else
    np_tile<OUT_F32, NpPipe256>(A, As, Ao, B, Bs, N, K, ti, lds, ab, out, bg);
}

// 128 x 512 tiles for experts of few rows each, 1 x 4 waves of 128 x 128
// (a sub-step decodes 4 + 4 fragments for 16 MFMAs); an expert's last tile
// multiplies only the 32-row groups that hold rows (with the DeepSeek-V3
// routing, median 88 rows per expert, 1.11x the routed rows instead of 1.33x).
template <bool OUT_F32, bool BIAS>
__global__ __launch_bounds__(256, 1) void k_gemm_nvfp4_wide(
    const uint8_t *__restrict__ A, const uint8_t *__restrict__ As,
    const float *__restrict__ Ao, const uint8_t *__restrict__ B,
    const uint8_t *__restrict__ Bs, const float *__restrict__ Bo, int64_t b_rps,
    const int64_t *__restrict__ offsets, int64_t G, int64_t N, int64_t K, int64_t ntn,
    void *__restrict__ out, const float *__restrict__ bias) {
  using W4 = Np<128, 512, 1, 4>;
  __shared__ __attribute__((aligned(16))) uint8_t lds[W4::LDS];
  __shared__ float ab[512];
  __shared__ int64_t sh[4];
  TileInfo ti;
  if (!lookup_row_tile<512, 128>(offsets, G, ntn, ti, sh)) return;
  for (int c = threadIdx.x; c < 512; c += 256) {  // alpha_b(n) = Bo[(g N + n) / b_rps]
    const int64_t col = ti.n0 + c;
    ab[c] = col < N ? Bo[(ti.g * N + col) / b_rps] : 0.0f;
  }
  __syncthreads();
  const int64_t rows = ti.row_end - ti.row0;
  const float *bg = BIAS ? bias + ti.g * N : nullptr;
  if (rows > 96)
    np_tile<OUT_F32, W4>(A, As, Ao, B, Bs, N, K, ti, lds, ab, out, bg);
  else if (rows > 64)
    np_tile<OUT_F32, Np<128, 512, 1, 3>>(A, As, Ao, B, Bs, N, K, ti, lds, ab, out, bg);
  else if (rows > 32)
    np_tile<OUT_F32, Np<128, 512, 1, 2>>(A, As, Ao, B, Bs, N, K, ti, lds, ab, out, bg);
  else
    np_tile<OUT_F32, Np<128, 512, 1, 1>>(A, As, Ao, B, Bs, N, K, ti, lds, ab, out, bg);
}

// ------------------------------------- NVFP4, persistent 128 x 512 tiles
// k_gemm_nvfp4_wide as a persistent kernel (bf16 output, no bias): one
// workgroup per CU walks its tiles (dealt as the tile list below says) as one
// unbroken stream of ring steps.  The ring refills run three
// steps ahead across tile boundaries (the loader moves on to the next tile
// when a refill reaches its step 0), together with that tile's outer scales
// (128 alpha_a and 512 alpha_b values, by DMA into one of two LDS buffers);
// a tile's output leaves by buffer stores issued after its last step (NPW_ST
// per lane, rows and columns outside the tile dropped by an out-of-range
// offset).  The waits count loads only (loads complete in order among
// themselves; a store, above all one with every lane out of range, need not
// keep its place in vmcnt), so the stores hold the next tile's first waits up
// only while they outnumber the younger loads still out.  Each workgroup
// keeps its CU, so neither the tile's prologue nor its stores wait for a
// workgroup to end and another to start.

template <int FI_>
using NpW = Np<128, 512, 1, FI_>;
constexpr int NPW_MAXT = 256;  // tiles per workgroup
constexpr int NPW_ST = 32;     // bf16 stores per lane per tile (4 x 4 fragments x 2)
constexpr int NPW_AL = 768;    // alpha floats per buffer: 128 rows, 512 columns, padding

// Exclusive prefix of v over the 256 threads (thread order) plus `carry`,
// which then grows by the 256 values' sum.  wsum: 4 shared slots.
__device__ __forceinline__ int32_t np_scan256(int32_t v, int32_t &carry, int32_t *wsum) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int32_t incl = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int32_t t = __shfl_up(incl, o, 64);
    if (lane >= o) incl += t;
  }
  if (lane == 63) wsum[wave] = incl;
  __syncthreads();
  int32_t before = carry, all = 0;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    before += w < wave ? wsum[w] : 0;
    all += wsum[w];
  }
  carry += all;
  __syncthreads();
  return before + incl - v;
}

// The outer scales of tile t by DMA: entry e = tid + 256 i (i = 0..2) of the
// buffer is alpha_a of row row0 + e (e < 128, clamped to the tile's rows) or
// alpha_b(n0 + e - 128) (clamped to column N - 1); entries 640.. repeat
// alpha_a of row row0.  abase: this wave's LDS address in the buffer.
__device__ __forceinline__ void npw_alpha_issue(const float *__restrict__ Ao,
                                                const float *__restrict__ Bo, int64_t b_rps,
                                                int64_t N, const QpTile &t, uint32_t abase) {
  int tid = threadIdx.x;
  asm volatile("" : "+v"(tid));
#pragma unroll
  for (int i = 0; i < 3; ++i) {
    const int e = tid + 256 * i;
    const float *src;
    if (e < 128) {
      src = Ao + min((int64_t)t.row0 + e, (int64_t)t.row_end - 1);
    } else if (e < 640) {
      const int64_t col = min((int64_t)t.n0 + (e - 128), N - 1);
      src = Bo + ((int64_t)t.g * N + col) / b_rps;
    } else {
      src = Ao + t.row0;
    }
    dma4(src, abase + (uint32_t)i * 1024u);
  }
}

// The tile's bf16 output: NPW_ST buffer stores per lane whatever the tile's
// fragment count (fragments i >= FI and cells outside the tile get an
// out-of-range offset); values as np_store scales them (binary64 product of
// the accumulator and alpha_a alpha_b, one rounding to binary32, then bf16).
template <class C>
__device__ __forceinline__ void npw_store(const v16f (&acc)[C::FI][C::FJ],
                                          __amdgpu_buffer_rsrc_t rs, const QpTile &t, int64_t N,
                                          const float *al) {
  static_assert(C::WM == 1 && C::FJ == 4, "1 x 4 waves of 128 x 128");
  typedef unsigned int u32x4 __attribute__((__vector_size__(16)));
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, h = lane >> 5, r32 = lane & 31;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int rl = 32 * i + r32;  // row within the tile
    const int64_t row = (int64_t)t.row0 + rl;
    const double aa = (double)al[rl];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        const int c0 = wave * C::WCOLS + 32 * j + 16 * p + 8 * h;  // column within the tile
        const int64_t col = (int64_t)t.n0 + c0;
        u32x4 w = {0u, 0u, 0u, 0u};
        uint32_t off = QP_OOB;
        if (i < C::FI) {
          const v16f &a = acc[i < C::FI ? i : 0][j];
          float lo[4], hi[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float x = a[8 * p + e], y = a[8 * p + 4 + e];
            const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(h ? x : y),
                                                             __float_as_uint(h ? x : y), false,
                                                             false);
            const float got = __uint_as_float(h ? sw[0] : sw[1]);
            lo[e] = h ? got : x;
            hi[e] = h ? y : got;
          }
          float v[8] = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
#pragma unroll
          for (int e = 0; e < 8; ++e) v[e] = (float)((double)v[e] * (aa * (double)al[128 + c0 + e]));
          w = u32x4{pk_bf16_rne(v[0], v[1]), pk_bf16_rne(v[2], v[3]), pk_bf16_rne(v[4], v[5]),
                    pk_bf16_rne(v[6], v[7])};
          if (row < t.row_end && col < N) off = (uint32_t)((row * N + col) * 2);
        }
        __builtin_amdgcn_raw_buffer_store_b128(w, rs, (int)off, 0, 0);
      }
    }
  }
}

// One tile of the persistent stream (C: its fragment count); slot: the ring
// slot of the tile's step 0 on entry, of the next tile's step 0 on exit.
template <class C>
__device__ __forceinline__ void npw_tile(NpSrc<C> &L, const QpTile *tl, int t, int S, int nk,
                                         int &slot, const uint8_t *lds, const NpLane &o,
                                         const uint8_t *__restrict__ A,
                                         const uint8_t *__restrict__ As,
                                         const float *__restrict__ Ao,
                                         const uint8_t *__restrict__ B,
                                         const uint8_t *__restrict__ Bs,
                                         const float *__restrict__ Bo, int64_t b_rps, int64_t N,
                                         int64_t K, uint32_t abase, const float *al,
                                         __amdgpu_buffer_rsrc_t rs) {
  constexpr int FI = C::FI, FJ = C::FJ;
  if (t > 0) {
    // own loads of this tile's step 0 done (the loads of its steps 1 and 2
    // may be pending: the count names loads only, which complete in order,
    // while the last tile's stores, some with every lane out of range, need
    // not hold their place); after the barrier every wave's are
    vm_wait<2 * C::OPS>();
    lgkm_wait0();
    wg_barrier();
  }
  NpHalf<C> R0, R1;
  NpWords<C> W;
  NpScales<C> S_;
  NpDec<C> X, Y;
  np_read_half<C, 0>(lds, slot, o, R0);
  np_read_half<C, 1>(lds, slot, o, R1);
  np_read_words<C>(lds, slot, o, W);
  np_scales<C, 0>(W, S_);
  np_dec<C, 0>(R0, S_, X);
  v16f acc[FI][FJ];
#pragma unroll
  for (int i = 0; i < FI; ++i)
#pragma unroll
    for (int j = 0; j < FJ; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
  for (int k = 0; k < nk; ++k) {
    // own loads of step k + 1 done (one step's refill may be pending)
    vm_wait<C::OPS>();
    lgkm_wait0();
    wg_barrier();
    const int nslot = slot == C::NSLOT - 1 ? 0 : slot + 1;
    // the refill: stream step t nk + k + NSLOT, i.e. step vk of tile vt
    // (nk >= NSLOT, so at most one tile ahead; counted, not divided, since a
    // division by the run-time nk costs a few dozen instructions a step);
    // past the end the last step again (in bounds; read, never multiplied)
    const int kv = k + C::NSLOT;
    const int vt = kv >= nk ? t + 1 : t, vk = kv >= nk ? kv - nk : kv;
    int rk = nk - 1;
    if (vt * nk + vk < S) {
      rk = vk;
      if (vk == 0) {  // the refills move on to tile vt, with its outer scales
        const QpTile tn = tl[vt];
        np_loader<C>(L, A, As, B, Bs, N, K, tn.g, tn.row0, tn.row_end, tn.n0);
        npw_alpha_issue(Ao, Bo, b_rps, N, tn, abase + (uint32_t)(vt & 1) * (NPW_AL * 4));
      }
    }
    np_step<C>(L, rk, slot, lds, o, nslot, acc, R0, R1, W, S_, X, Y);
    slot = nslot;
  }
  npw_store<C>(acc, rs, tl[t], N, al);
}

__global__ __launch_bounds__(256, 1) void k_gemm_nvfp4_wide_p(
    const uint8_t *__restrict__ A, const uint8_t *__restrict__ As,
    const float *__restrict__ Ao, const uint8_t *__restrict__ B,
    const uint8_t *__restrict__ Bs, const float *__restrict__ Bo, int64_t b_rps,
    const int64_t *__restrict__ offsets, int64_t G, int64_t N, int64_t K, int64_t ntn,
    void *__restrict__ out, uint32_t out_bytes) {
  using W4 = NpW<4>;
  __shared__ __attribute__((aligned(16))) uint8_t lds[W4::LDS];
  __shared__ __attribute__((aligned(16))) float alpha[2 * NPW_AL];
  __shared__ QpTile tl[NPW_MAXT];
  __shared__ int32_t wsum[4], nt_sh;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h = lane >> 5, r32 = lane & 31;

  // ---- tile list.  Row tiles in four classes by the fragments they
  // multiply (a full tile or a tail of 97..127 rows: 4; tails of 65..96: 3;
  // 33..64: 2; 1..32: 1), heaviest class first, experts in order within a
  // class; row tile R goes to XCD R % 8 with its column tiles (so they share
  // that XCD's L2), and an XCD deals its tiles, in that order, round-robin
  // to its workgroups: every workgroup gets a like mix of heavy and light
  // tiles.  pre[c (G + 1) + g]: row tiles of class 4 - c before expert g.
  int32_t *pre = reinterpret_cast<int32_t *>(lds);  // 4 (G + 1) entries (checked on the host)
  {
    int32_t carry[4] = {0, 0, 0, 0};
    for (int64_t b0 = 0; b0 < G; b0 += 256) {
      const int64_t g = b0 + tid;
      const int64_t rows = g < G ? offsets[g + 1] - offsets[g] : 0;
      const int32_t full = (int32_t)(rows / 128), tc = (int32_t)((rows % 128 + 31) / 32);
      const int32_t v[4] = {full + (tc == 4), tc == 3, tc == 2, tc == 1};
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int32_t x = np_scan256(v[c], carry[c], wsum);
        if (g < G) pre[c * (G + 1) + g] = x;
      }
    }
    if (tid == 0) {
#pragma unroll
      for (int c = 0; c < 4; ++c) pre[c * (G + 1) + G] = carry[c];
    }
  }
  __syncthreads();
  {
    int32_t cnt[4], nrt = 0;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      cnt[c] = pre[c * (G + 1) + G];
      nrt += cnt[c];
    }
    const int x = (int)(blockIdx.x % 8), w = (int)(blockIdx.x / 8), nw = (int)(gridDim.x / 8);
    const int64_t nq = (int64_t)(nrt > x ? (nrt - x + 7) / 8 : 0) * ntn;  // this XCD's tiles
    const int nt = nq > w ? (int)((nq - w + nw - 1) / nw) : 0;
    if (tid == 0) nt_sh = min(nt, NPW_MAXT);
    for (int k = tid; k < nt && k < NPW_MAXT; k += 256) {
      const int64_t q = w + (int64_t)k * nw;
      const int32_t R = (int32_t)(8 * (q / ntn) + x);
      int c = 0;
      int32_t r = R;
      while (c < 3 && r >= cnt[c]) r -= cnt[c++];
      const int32_t *pc = pre + c * (G + 1);
      int a = 0, bb = (int)G;  // largest g with pc[g] <= r (pc[G] > r)
      while (bb - a > 1) {
        const int m = (a + bb) >> 1;
        if (pc[m] <= r) a = m; else bb = m;
      }
      const int64_t rows = offsets[a + 1] - offsets[a];
      QpTile t;
      t.g = a;
      t.row0 = (int32_t)(offsets[a] + 128 * (c == 0 ? (int64_t)(r - pc[a]) : rows / 128));
      t.row_end = (int32_t)offsets[a + 1];
      t.n0 = (int32_t)((q % ntn) * 512);
      tl[k] = t;
    }
  }
  __syncthreads();  // the tile list is complete and pre is no longer read
  const int nt = nt_sh;
  if (nt == 0) return;
  const int nk = (int)(K / 128);  // >= 3
  const int S = nt * nk;
  const __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc(out, (short)0, (int)out_bytes, 0x00020000);
  NpSrc<W4> L;
  L.dst = __builtin_amdgcn_readfirstlane(lds_addr(lds) + (uint32_t)wave * 1024u);
  L.sdst = __builtin_amdgcn_readfirstlane(lds_addr(lds) + W4::SC + (uint32_t)wave * 256u);
  const uint32_t abase = __builtin_amdgcn_readfirstlane(lds_addr(alpha) + (uint32_t)wave * 256u);
  NpLane o;
  {
    const int ra = r32, rb = wave * W4::WCOLS + r32;
    o.a0 = mx3_off(ra, 2 * h);
    o.a1 = mx3_off(ra, 2 * h + 1);
    o.b0 = W4::TMR * 64 + mx3_off(rb, 2 * h);
    o.b1 = W4::TMR * 64 + mx3_off(rb, 2 * h + 1);
    o.sa = W4::SC + ra * 8 + 4 * h;
    o.sb = W4::SC + (W4::TMR + rb) * 8 + 4 * h;
  }
  // prologue: tile 0's outer scales and its steps 0 .. 2
  {
    const QpTile t0 = tl[0];
    np_loader<W4>(L, A, As, B, Bs, N, K, t0.g, t0.row0, t0.row_end, t0.n0);
    npw_alpha_issue(Ao, Bo, b_rps, N, t0, abase);
#pragma unroll
    for (int s = 0; s < W4::NSLOT; ++s) np_issue<W4>(L, s, s);
  }
  vm_wait<(W4::NSLOT - 1) * W4::OPS>();  // the outer scales and step 0
  lgkm_wait0();
  wg_barrier();
  int slot = 0;
  for (int t = 0; t < nt; ++t) {
    const int rows = tl[t].row_end - tl[t].row0;
    const float *al = alpha + (t & 1) * NPW_AL;
    if (rows > 96)
      npw_tile<W4>(L, tl, t, S, nk, slot, lds, o, A, As, Ao, B, Bs, Bo, b_rps, N, K, abase, al,
                   rs);
    else if (rows > 64)
      npw_tile<NpW<3>>(L, tl, t, S, nk, slot, lds, o, A, As, Ao, B, Bs, Bo, b_rps, N, K, abase,
                       al, rs);
    else if (rows > 32)
      npw_tile<NpW<2>>(L, tl, t, S, nk, slot, lds, o, A, As, Ao, B, Bs, Bo, b_rps, N, K, abase,
                       al, rs);
    else
      npw_tile<NpW<1>>(L, tl, t, S, nk, slot, lds, o, A, As, Ao, B, Bs, Bo, b_rps, N, K, abase,
                       al, rs);
  }
  vm_wait<0>();  // stores done and no load still targets this workgroup's LDS
}

// ------------------------------------------- NVFP4 FC2 with online amax
// "miniTE technical report", 5.6: FC2 consumes the activation P (the
// weighted SwiGLU output, bf16) K-tile by K-tile, before a row's full
// maximum is known.  Each row keeps a running maximum gamax; K-tile i of the
// row is encoded (1x16 E4M3 block scales, E2M1 codes) under the running outer
// scale gs = gamax / 2688, multiplied block-scaled with W2 (the product
// leaves gs out), and the accumulator of the earlier tiles is first moved to
// the new scale, O = O (gs_prev / gs) + dO_i; Y = O gs_prev alpha_W2.  A row
// whose maximum is still zero contributes nothing and keeps gs_prev (its
// codes and block scales are zero).
//
// The multiply is the NVFP4 grouped GEMM's step and ring (128 x 256 tiles on
// 2 x 2 waves) with the A part of each ring slot written by the workgroup:
// the ring carries W2 only, and P's 128-wide tiles come by DMA through a
// two-slot LDS ring of their own.  Step kt encodes tile kt + 2 into ring slot
// (kt + 2) % 3, whose previous step was read during step kt - 2, and then
// multiplies step kt.  Every column tile of a row block encodes the same P
// tiles the same way, so all of them agree on each gs without exchanging it.

using NpOn = Np<128, 256, 2, 2, false>;
constexpr int NPO_PL = 8;               // P-ring loads per lane per tile
constexpr int NPO_PSLOT = 128 * 256;    // bytes of one P tile (128 rows x 128 bf16)


// Running state of the rows tid / 8 + 32 j (j = 0..3) of the thread's blocks;
// the 8 threads of a row hold the same values.  rc: the encoding constants of
// the running maximum (recomputed only when it grows).
struct NpoRows {
  uint32_t gam[4];  // running maximum (bf16 magnitude bits)
  Nvfp4Row rc[4];   // rc.s_g: outer scale after the last tile with a non-zero maximum (0 before)
};

// Maximum over the 8 lanes 8 (lane / 8) .. of a wave: quad swaps by 1 and 2,
// then the mirror within 8 lanes (lane i and 7 - i).
__device__ __forceinline__ uint32_t max8_lanes(uint32_t v) {
  v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x141, 0xF, 0xF, false));
  return v;
}

// P tile t into P-ring slot ps: load i = 2 j + hb of thread tid fetches
// 16 bytes of row tid / 8 + 32 j (clamped to the tile's rows), bytes
// 16 (8 hb + tid % 8) .. of the tile (each load covers one 128-byte half of 8
// rows), to LDS chunk 256 i + tid.
__device__ __forceinline__ void npo_issue_p(const uint16_t *Pt, int64_t K, int rows_a, int t,
                                            uint32_t pdst, int ps) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int i = 0; i < NPO_PL; ++i) {
    const int r = min(tid / 8 + 32 * (i >> 1), rows_a - 1);
    const uint16_t *src = Pt + (int64_t)r * K + 128 * t + 8 * (8 * (i & 1) + (tid & 7));
    dma16(src, pdst + (uint32_t)(ps * NPO_PSLOT + i * 4096));
  }
}

// Encode P tile t (P-ring slot ps) into the A part of ring slot `sp`: thread
// tid takes the 1x16 blocks (row tid / 8 + 32 j, block tid % 8).  The tile's
// row maximum joins the running one; gs and the ratio gs_prev / gs (1 while
// the maximum is zero) go to `ratio` and `gsf` by row.  With q_out, the codes
// and block scales of the tile's rows are also written to memory.
__device__ __forceinline__ void npo_encode(const uint8_t *pring, int ps, uint8_t *sp,
                                           float *ratio, float *gsf, NpoRows &st, int t,
                                           int rows_a, int64_t row0, int64_t K,
                                           uint8_t *__restrict__ q_out,
                                           uint8_t *__restrict__ sb_out) {
  const int tid = threadIdx.x, blk = tid & 7;
  const uint8_t *pb = pring + ps * NPO_PSLOT;
  uint32_t w[4][8], m[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    // chunks 2 blk, 2 blk + 1 of row tid / 8 + 32 j: load 2 j + blk / 4,
    // lanes 8 (tid / 8) + 2 (blk % 4) and the next
    const uint8_t *src = pb + 4096 * (2 * j + (blk >> 2)) + 16 * (8 * (tid >> 3) + 2 * (blk & 3));
    const uint4 v0 = *reinterpret_cast<const uint4 *>(src);
    const uint4 v1 = *reinterpret_cast<const uint4 *>(src + 16);
    w[j][0] = v0.x; w[j][1] = v0.y; w[j][2] = v0.z; w[j][3] = v0.w;
    w[j][4] = v1.x; w[j][5] = v1.y; w[j][6] = v1.z; w[j][7] = v1.w;
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    uint32_t mm = 0;
#pragma unroll
    for (int k = 0; k < 8; ++k) mm = pk_max_u16(mm, w[j][k] & 0x7FFF7FFFu);
    m[j] = max8_lanes(max(mm & 0xFFFFu, mm >> 16));
  }
  float rt[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const bool grew = m[j] > st.gam[j];
    rt[j] = 1.0f;
    if (__builtin_amdgcn_ballot_w64(grew) != 0) {
      if (grew) {
        st.gam[j] = m[j];
        const Nvfp4Row rc = nvfp4_row(__uint_as_float(m[j] << 16));
        rt[j] = __fdiv_rn(st.rc[j].s_g, rc.s_g);
        st.rc[j] = rc;
      }
    }
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int r = tid / 8 + 32 * j;
    uint32_t sbc;
    const uint2 packed = nvfp4_block(w[j], st.rc[j], &sbc);
    *reinterpret_cast<uint2 *>(sp + r * 64 + (((blk >> 1) ^ (r >> 2)) & 3) * 16 + 8 * (blk & 1)) =
        packed;
    sp[NpOn::SC + r * 8 + blk] = (uint8_t)sbc;
    if (blk == 0) {
      ratio[r] = rt[j];
      gsf[r] = st.rc[j].s_g;
    }
    if (q_out && r < rows_a) {
      const int64_t row = row0 + r;
      *reinterpret_cast<uint2 *>(q_out + row * (K / 2) + 64 * t + 8 * blk) = packed;
      sb_out[row * (K / 16) + 8 * t + blk] = (uint8_t)sbc;
    }
  }
}

// Move each accumulator row to the step's outer scale (skipped for a
// fragment whose 32 rows all keep theirs).
template <class C>
__device__ __forceinline__ void npo_rescale(const float *ratio, int wm, int r32,
                                            v16f (&acc)[C::FI][C::FJ]) {
#pragma unroll
  for (int i = 0; i < C::FI; ++i) {
    const float rt = ratio[wm * C::WROWS + 32 * i + r32];
    if (__builtin_amdgcn_ballot_w64(rt != 1.0f) != 0) {
#pragma unroll
      for (int j = 0; j < C::FJ; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[i][j][e] *= rt;
    }
  }
}

// Y [M, N] = online-amax FC2 of P [M, K] bf16 with W2 [G N, K] NVFP4
// (alpha_W2(n) = Bo[(g N + n) / b_rps]); K % 256 == 0.  gs_out: each row's
// final outer scale; q_out / sb_out: P's codes and block scales as encoded
// (written by the first column tile).
template <bool OUT_F32>
__global__ __launch_bounds__(256, 1) void k_gemm_nvfp4_online(
    const uint16_t *__restrict__ P, const uint8_t *__restrict__ B,
    const uint8_t *__restrict__ Bs, const float *__restrict__ Bo, int64_t b_rps,
    const int64_t *__restrict__ offsets, int64_t G, int64_t N, int64_t K, int64_t ntn,
    void *__restrict__ out, float *__restrict__ gs_out, uint8_t *__restrict__ q_out,
    uint8_t *__restrict__ sb_out) {
  using C = NpOn;
  constexpr int FI = C::FI, FJ = C::FJ;
  __shared__ __attribute__((aligned(16))) uint8_t lds[C::LDS];
  __shared__ __attribute__((aligned(16))) uint8_t pring[2 * NPO_PSLOT];
  __shared__ float ratio[C::NSLOT][C::TMR];
  __shared__ float gsf[C::TMR];
  __shared__ float ab[C::TN];
  __shared__ int64_t sh[4];
  TileInfo ti;
  if (!lookup_row_tile<C::TN, C::TMR>(offsets, G, ntn, ti, sh)) return;
  {  // the tile's column scales alpha_W2(n)
    const int64_t col = ti.n0 + threadIdx.x;
    ab[threadIdx.x] = col < N ? Bo[(ti.g * N + col) / b_rps] : 0.0f;
  }
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int h = lane >> 5, r32 = lane & 31;
  const uint32_t KD = (uint32_t)(K / 2), KS = (uint32_t)(K / 16);
  const int rows_a = (int)min(ti.row_end - ti.row0, (int64_t)C::TMR);
  const int rows_b = (int)min(N - ti.n0, (int64_t)C::TN);
  NpSrc<C> L;
  L.Ab = nullptr;
  L.Asb = nullptr;
  L.Bb = B + (ti.g * N + ti.n0) * (int64_t)KD;
  L.Bsb = Bs + (ti.g * N + ti.n0) * (int64_t)KS;
  L.dst = __builtin_amdgcn_readfirstlane(lds_addr(lds) + (uint32_t)wave * 1024u);
  L.sdst = __builtin_amdgcn_readfirstlane(lds_addr(lds) + C::SC + (uint32_t)wave * 256u);
#pragma unroll
  for (int i = 0; i < C::CA; ++i) L.oa[i] = 0;
#pragma unroll
  for (int i = 0; i < C::CB; ++i) {
    const int c = tid + 256 * i, r = c >> 2, k = (c & 3) ^ ((r >> 2) & 3);
    L.ob[i] = (uint32_t)min(r, rows_b - 1) * KD + 16u * k;
  }
#pragma unroll
  for (int i = 0; i < C::NS; ++i) {  // only i >= NS0 (the B rows) are loaded
    const int d = tid + 256 * i, r = d >> 1, half = d & 1;
    L.os[i] = r < C::TMR ? 0u : (uint32_t)min(r - C::TMR, rows_b - 1) * KS + 4u * half;
  }
  NpLane o;
  {
    const int ra = wm * C::WROWS + r32, rb = wn * C::WCOLS + r32;
    o.a0 = mx3_off(ra, 2 * h);
    o.a1 = mx3_off(ra, 2 * h + 1);
    o.b0 = C::TMR * 64 + mx3_off(rb, 2 * h);
    o.b1 = C::TMR * 64 + mx3_off(rb, 2 * h + 1);
    o.sa = C::SC + ra * 8 + 4 * h;
    o.sb = C::SC + (C::TMR + rb) * 8 + 4 * h;
  }
  v16f acc[FI][FJ];
#pragma unroll
  for (int i = 0; i < FI; ++i)
#pragma unroll
    for (int j = 0; j < FJ; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  const uint16_t *Pt = P + ti.row0 * K;
  const uint32_t pdst = __builtin_amdgcn_readfirstlane(lds_addr(pring) + (uint32_t)wave * 1024u);
  uint8_t *qo = ti.n0 == 0 ? q_out : nullptr;
  NpoRows st;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    st.gam[j] = 0;
    st.rc[j] = nvfp4_row(0.0f);  // s_g = 0: the zero row's encoding
  }
  const int nk = (int)(K / 128);  // even, >= 2
  // prologue: W2 steps 0..2, P tiles 0 and 1 encoded into slots 0 and 1,
  // P tile 2 requested
#pragma unroll
  for (int s = 0; s < C::NSLOT; ++s) np_issue<C>(L, min(s, nk - 1), s);
  npo_issue_p(Pt, K, rows_a, 0, pdst, 0);
  npo_issue_p(Pt, K, rows_a, 1, pdst, 1);
  vm_wait<NPO_PL>();  // all but P tile 1
  wg_barrier();
  npo_encode(pring, 0, lds, ratio[0], gsf, st, 0, rows_a, ti.row0, K, qo, sb_out);
  vm_wait<0>();
  lgkm_wait0();
  wg_barrier();  // P tile 1 landed; P slot 0 read by every wave
  npo_encode(pring, 1, lds + C::SLOT, ratio[1], gsf, st, 1, rows_a, ti.row0, K, qo, sb_out);
  npo_issue_p(Pt, K, rows_a, min(2, nk - 1), pdst, 0);
  lgkm_wait0();
  wg_barrier();
  NpHalf<C> R0, R1;
  NpWords<C> W;
  NpScales<C> S;
  NpDec<C> X, Y;
  np_read_half<C, 0>(lds, 0, o, R0);
  np_read_half<C, 1>(lds, 0, o, R1);
  np_read_words<C>(lds, 0, o, W);
  np_scales<C, 0>(W, S);
  np_dec<C, 0>(R0, S, X);
  int slot = 0;
  for (int kt = 0; kt < nk; ++kt) {
    // own loads of P tile kt + 2 and of W2 step kt + 1 done (only W2 step
    // kt + 2, requested during step kt - 1, may be pending; at kt = 0 P tile
    // 2 is the newest load); after the barrier every wave's are, and P slot
    // (kt + 1) % 2 and ring slot (kt + 2) % 3 are no longer read
    if (kt == 0)
      vm_wait<0>();
    else
      vm_wait<C::OPS>();
    lgkm_wait0();
    wg_barrier();
    const int nslot = slot == C::NSLOT - 1 ? 0 : slot + 1;
    npo_issue_p(Pt, K, rows_a, min(kt + 3, nk - 1), pdst, (kt + 1) & 1);
    if (kt + 2 < nk) {
      const int es = nslot == C::NSLOT - 1 ? 0 : nslot + 1;  // (kt + 2) % 3
      npo_encode(pring, kt & 1, lds + es * C::SLOT, ratio[es], gsf, st, kt + 2, rows_a, ti.row0,
                 K, qo, sb_out);
    }
    npo_rescale<C>(ratio[slot], wm, r32, acc);
    // past the last step the reads take the slot's repeated last step (in
    // bounds; decoded, never multiplied)
    np_step<C>(L, min(kt + C::NSLOT, nk - 1), slot, lds, o, nslot, acc, R0, R1, W, S, X, Y);
    slot = nslot;
  }
  vm_wait<0>();
#pragma unroll
  for (int i = 0; i < FI; ++i)
#pragma unroll
    for (int j = 0; j < FJ; ++j)
      np_store<OUT_F32, true>(acc[i][j], out, N, ti.row0, ti.row_end, ti.n0,
                              wm * C::WROWS + 32 * i, wn * C::WCOLS + 32 * j, gsf, ab);
  if (gs_out && ti.n0 == 0 && tid < rows_a) gs_out[ti.row0 + tid] = gsf[tid];
}

// The same FC2 split into two kernels: the encoding of P does not depend on the
// output column, so one pass encodes every routed row once (the running
// maximum, gs, E4M3 block scales and E2M1 codes of each 128-wide K-tile, as
// npo_encode computes them, and each tile's gs_prev / gs), and the GEMM then
// reads the codes like any NVFP4 operand and moves its accumulator rows by
// the stored ratios before each step.  The accumulation and the epilogue
// (the final gs as the row's outer scale) are those of the one-kernel path,
// whose column tiles each encode P again.
constexpr int NPO_MAX_NK = 32;  // K / 128 ratios of a tile row held in LDS

// Encode pass: 8 lanes per row, lane b taking the 1x16 block b of every
// 128-wide tile, in K order.  q [rows, K/2], sb [rows, K/16], gs [rows],
// ratio [rows, K/128] for the rows 0 .. offsets[G]-1.
__global__ __launch_bounds__(256) void k_online_encode_nvfp4(
    const uint16_t *__restrict__ P, const int64_t *__restrict__ offsets, int64_t G, int64_t K,
    uint8_t *__restrict__ q, uint8_t *__restrict__ sb, float *__restrict__ gs,
    float *__restrict__ ratio) {
  const int64_t rows = offsets[G];
  const int64_t row = (int64_t)blockIdx.x * 32 + (threadIdx.x >> 3);
  if ((int64_t)blockIdx.x * 32 >= rows) return;  // whole workgroup: no lane of it has a row
  const int blk = threadIdx.x & 7;
  const bool ok = row < rows;
  const uint16_t *pr = P + min(row, rows - 1) * K + 16 * blk;
  const int nk = (int)(K / 128);
  uint32_t gam = 0;
  Nvfp4Row rc = nvfp4_row(0.0f);  // s_g = 0 while the maximum is zero
  // tiles t + 1 and t + 2 are loaded while tile t is encoded (nk >= 2; a
  // load past the last tile re-reads the last one and is not used)
  uint4 a0 = *reinterpret_cast<const uint4 *>(pr), a1 = *reinterpret_cast<const uint4 *>(pr + 8);
  uint4 b0 = *reinterpret_cast<const uint4 *>(pr + 128),
        b1 = *reinterpret_cast<const uint4 *>(pr + 128 + 8);
  for (int t = 0; t < nk; ++t) {
    const uint4 v0 = a0, v1 = a1;
    a0 = b0;
    a1 = b1;
    const int tn = min(t + 2, nk - 1);
    b0 = *reinterpret_cast<const uint4 *>(pr + 128 * tn);
    b1 = *reinterpret_cast<const uint4 *>(pr + 128 * tn + 8);
    const uint32_t w[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
    uint32_t mm = 0;
#pragma unroll
    for (int k = 0; k < 8; ++k) mm = pk_max_u16(mm, w[k] & 0x7FFF7FFFu);
    const uint32_t m = max8_lanes(max(mm & 0xFFFFu, mm >> 16));
    float rt = 1.0f;
    if (m > gam) {
      gam = m;
      const Nvfp4Row n = nvfp4_row(__uint_as_float(m << 16));
      rt = __fdiv_rn(rc.s_g, n.s_g);
      rc = n;
    }
    uint32_t sbc;
    const uint2 packed = nvfp4_block(w, rc, &sbc);
    if (ok) {
      *reinterpret_cast<uint2 *>(q + row * (K / 2) + 64 * t + 8 * blk) = packed;
      sb[row * (K / 16) + 8 * t + blk] = (uint8_t)sbc;
      if (blk == 0) ratio[row * nk + t] = rt;
    }
  }
  if (ok && blk == 0) gs[row] = rc.s_g;
}

// GEMM pass: the pipelined NVFP4 kernel's 128 x 256 tiles (2 x 2 waves,
// the one-kernel path's shape) with the per-step rescale; A = the encode
// pass's codes and block scales, its outer scale the final gs.  (256-row
// tiles keep 256 accumulators per lane, which the rescale's multiplies
// would have to move through VGPRs: 272 spilled registers.)
template <bool OUT_F32>
__global__ __launch_bounds__(256, 1) void k_gemm_nvfp4_rescale(
    const uint8_t *__restrict__ A, const uint8_t *__restrict__ As,
    const float *__restrict__ Ao, const uint8_t *__restrict__ B,
    const uint8_t *__restrict__ Bs, const float *__restrict__ Bo, int64_t b_rps,
    const int64_t *__restrict__ offsets, int64_t G, int64_t N, int64_t K, int64_t ntn,
    void *__restrict__ out, const float *__restrict__ ratio) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[NpPipe128::LDS];
  __shared__ float rl[NPO_MAX_NK * 128];
  __shared__ float ab[256];
  __shared__ int64_t sh[4];
  TileInfo ti;
  if (!lookup_row_tile<256, 128>(offsets, G, ntn, ti, sh)) return;
  {
    const int64_t col = ti.n0 + threadIdx.x;
    ab[threadIdx.x] = col < N ? Bo[(ti.g * N + col) / b_rps] : 0.0f;
  }
  __syncthreads();
  np_tile<OUT_F32, NpPipe128>(A, As, Ao, B, Bs, N, K, ti, lds, ab, out, nullptr, ratio, rl);
}

// ------------------------------------------------------------------ launch

// K = 0: the product over an empty contraction is zero, so rows 0 ..
// offsets[G]-1 of Y [M, N] (element size esize) are cleared and nothing is
// read.  The pipelined kernels assume at least one contraction step; this
// keeps every K = 0 call away from them.
__global__ __launch_bounds__(256) void k_zero_rows(const int64_t *__restrict__ offsets, int64_t G,
                                                   int64_t N, int esize, void *__restrict__ out) {
  const int64_t bytes = offsets[G] * N * esize;  // a multiple of 2; out 16-byte aligned
  uint16_t *o = static_cast<uint16_t *>(out);
  const int64_t n = bytes / 2;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * 256)
    o[i] = 0;
}

// K = 0 with a bias: Y[m, :] = bias[g(m), :] for the routed rows (one wave
// per row; g(m) by binary search of the offsets).
__global__ __launch_bounds__(256) void k_bias_rows(const int64_t *__restrict__ offsets, int64_t G,
                                                   int64_t N, const float *__restrict__ bias,
                                                   int out_f32, void *__restrict__ out) {
  const int64_t M = offsets[G];
  for (int64_t m = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6); m < M;
       m += (int64_t)gridDim.x * 4) {
    int64_t lo = 0, hi = G - 1;  // the last group g with offsets[g] <= m
    while (lo < hi) {
      const int64_t mid = (lo + hi + 1) / 2;
      if (offsets[mid] <= m) lo = mid; else hi = mid - 1;
    }
    const float *b = bias + lo * N;
    for (int64_t n = threadIdx.x & 63; n < N; n += 64) {
      if (out_f32)
        static_cast<float *>(out)[m * N + n] = b[n];
      else
        static_cast<uint16_t *>(out)[m * N + n] = (uint16_t)f32_to_bf16_rne(b[n]);
    }
  }
}

static int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Persistent MXFP8 grid: one workgroup per CU (a multiple of 8, one range
// of tiles per XCD), fewer when there are fewer tiles.
static int64_t qp_grid(int64_t G, int64_t M, int64_t N) {
  const int64_t tiles_ub = (cdiv(M, 256) + G) * cdiv(N, 256);
  const int64_t cus = resident_workgroups((const void *)k_gemm_mxfp8_qp<false, false>, 512, 0);
  return max((int64_t)8, min(cdiv(cus, 8) * 8, cdiv(tiles_ub, 8) * 8));
}

// The persistent kernel's limits: the expert tile counts fit the ring's LDS
// for the scan, every workgroup's tiles fit its tile list, the output is
// below 2^31 bytes (its store offsets and the dropped offset), and rows are
// whole 16-byte store vectors.
static bool qp_fits(int64_t G, int64_t M, int64_t N, int64_t K, int esize) {
  (void)K;
  if ((G + 1) * 4 > Mq<256>::LDS) return false;
  if ((N * esize) % 16) return false;
  if (M * N * esize >= (int64_t)QP_OOB) return false;
  const int64_t tiles_ub = (cdiv(M, 256) + G) * cdiv(N, 256);
  const int64_t nw = qp_grid(G, M, N) / 8;
  return cdiv(cdiv(tiles_ub, 8), nw) <= QP_MAXT;
}

// Persistent NVFP4 grid: one workgroup per CU (a multiple of 8), fewer when
// there are fewer tiles; its limits: the expert tile counts fit the ring's
// LDS for the scan, every workgroup's tiles fit its list, the bf16 output is
// below 2^31 bytes (store offsets and the dropped offset), whole 16-byte
// output vectors, and at least 3 steps per tile (the refills run 3 ahead).
static int64_t npw_tiles_ub(int64_t G, int64_t M, int64_t N) {
  return (cdiv(M, 128) + G) * cdiv(N, 512);
}
static int64_t npw_grid(int64_t G, int64_t M, int64_t N) {
  const int64_t cus = resident_workgroups((const void *)k_gemm_nvfp4_wide_p, 256, 0);
  return max((int64_t)8, min(cdiv(cus, 8) * 8, cdiv(npw_tiles_ub(G, M, N), 8) * 8));
}
static bool npw_fits(int64_t G, int64_t M, int64_t N, int64_t K) {
  if (4 * (G + 1) * 4 > NpW<4>::LDS) return false;
  if (N % 8 || K / 128 < 3) return false;
  if (M * N * 2 >= (int64_t)QP_OOB) return false;
  const int64_t nw = npw_grid(G, M, N) / 8;
  return cdiv(cdiv(cdiv(M, 128) + G, 8) * cdiv(N, 512), nw) <= NPW_MAXT;
}

int64_t grouped_gemm_workspace_bytes(int fmt, int kind) {
  return fmt == 1 && kind == 2 ? 4 : 0;
}

// The persistent weight-gradient kernel: one workgroup per CU (a multiple
// of 8, so that every XCD holds the same number of ranks).
static int64_t mwq_grid(int64_t tiles) {
  const int64_t cus = resident_workgroups((const void *)k_gemm_mxfp8_wgrad_qp<true, true>, 512, 0);
  return max((int64_t)8, min(cdiv(cus, 8) * 8, cdiv(tiles, 8) * 8));
}

// Its limits: the per-expert tables fit LDS, buffer offsets of every operand,
// scale array and expert output below 2^31 (and the dropped offset), scale
// arrays that end on a 4-byte word (no aligned word reaches past them),
// 16-byte operand and output rows and pointers, 4-byte scale pointers.
static bool mwq_fits(const void *A, const void *As, const void *B, const void *Bs,
                     const void *out, int64_t G, int64_t M, int64_t N, int64_t K, int esize) {
  const int64_t lim = (int64_t)QP_OOB - 4096;
  if (G > MW_MAXG) return false;
  if (N * M >= lim || K * M >= lim || N * K * esize >= lim) return false;
  if (G * cdiv(N, 256) * cdiv(K, 256) >= lim) return false;
  if ((N * (M / 32)) % 4 || (K * (M / 32)) % 4) return false;
  if ((K * esize) % 16) return false;
  if (((uintptr_t)A | (uintptr_t)B | (uintptr_t)out) % 16 || ((uintptr_t)As | (uintptr_t)Bs) % 4)
    return false;
  return true;
}

hipError_t launch_grouped_gemm(int fmt, int kind, const void *a, const uint8_t *a_scale,
                               const float *a_outer, const void *b, const uint8_t *b_scale,
                               const float *b_outer, int64_t b_rows_per_scale,
                               const int64_t *offsets, int64_t G, int64_t M, int64_t N,
                               int64_t K, void *out, int out_fp32, const float *bias,
                               uint32_t *ctr, hipStream_t st) {
  if (G == 0 || N == 0) return hipSuccess;
  // kernels with a compile-time bias flag: <OUT_F32, BIAS> picked at run time
#define PQM_FB(KERN, GRID, BLOCK, ...)                                                  \
  do {                                                                                 \
    if (out_fp32) {                                                                    \
      if (bias) hipLaunchKernelGGL((KERN<true, true>), GRID, BLOCK, 0, st, __VA_ARGS__); \
      else hipLaunchKernelGGL((KERN<true, false>), GRID, BLOCK, 0, st, __VA_ARGS__);     \
    } else {                                                                           \
      if (bias) hipLaunchKernelGGL((KERN<false, true>), GRID, BLOCK, 0, st, __VA_ARGS__); \
      else hipLaunchKernelGGL((KERN<false, false>), GRID, BLOCK, 0, st, __VA_ARGS__);    \
    }                                                                                  \
  } while (0)
  const int64_t U32 = (int64_t)1 << 32;  // the pipelined kernels' per-panel byte offsets
  if (K == 0 && kind != 2) {  // FPROP / DGRAD over an empty contraction: Y = 0 (+ bias)
    if (M == 0) return hipSuccess;
    if (bias) {
      hipLaunchKernelGGL(k_bias_rows, dim3((unsigned)min(cdiv(M, 4), (int64_t)65536)), dim3(256),
                         0, st, offsets, G, N, bias, out_fp32, out);
      return hipGetLastError();
    }
    const int64_t n = M * N / 2 + 1;
    const unsigned grid = (unsigned)min(cdiv(n, 256), (int64_t)8192);
    hipLaunchKernelGGL(k_zero_rows, dim3(grid), dim3(256), 0, st, offsets, G, N,
                       out_fp32 ? 4 : 2, out);
    return hipGetLastError();
  }
  if (fmt == 3) {  // block-scaled FP8 forward
    if (M == 0) return hipSuccess;
    if (K % 128 || K / 128 > FB_MAX_KB || N % 128) return hipErrorNotSupported;
    const uint8_t *A = static_cast<const uint8_t *>(a), *B = static_cast<const uint8_t *>(b);
    const int64_t ntn_b = cdiv(N, 256);
    const dim3 grid_b((unsigned)(cdiv((cdiv(M, FB_TM) + G) * ntn_b, 8) * 8));
    PQM_FB(k_gemm_fp8_block, grid_b, dim3(256), A, a_outer, B, b_outer, offsets, G, N, K, ntn_b,
           out, bias);
    return hipGetLastError();
  }
  if (fmt == 1 && kind == 2) {  // WGRAD (MXFP8, column-wise copies)
    if (K == 0) return hipSuccess;
    if (M % 32 || M * 256 + 4096 >= U32) return hipErrorNotSupported;
    const int64_t ntm = cdiv(N, 256), ntn = cdiv(K, 256);
    const uint8_t *A = static_cast<const uint8_t *>(a), *B = static_cast<const uint8_t *>(b);
    if (mwq_fits(A, a_scale, B, b_scale, out, G, M, N, K, out_fp32 ? 4 : 2)) {
      const dim3 grid_p((unsigned)mwq_grid(G * ntm * ntn));
      const int32_t g32 = (int32_t)G, m32 = (int32_t)ntm, n32 = (int32_t)ntn;
      if (ctr) hipLaunchKernelGGL(k_zero_u32, dim3(1), dim3(1), 0, st, ctr);
#define PQM_MWQ(F32, DYN)                                                                      \
  hipLaunchKernelGGL((k_gemm_mxfp8_wgrad_qp<F32, DYN>), grid_p, dim3(512), 0, st, A, a_scale, B, \
                     b_scale, offsets, g32, M, N, K, m32, n32, out, ctr)
      if (out_fp32) {
        if (ctr) PQM_MWQ(true, true);
        else PQM_MWQ(true, false);
      } else {
        if (ctr) PQM_MWQ(false, true);
        else PQM_MWQ(false, false);
      }
#undef PQM_MWQ
      return hipGetLastError();
    }
    const dim3 grid((unsigned)(cdiv(G * ntm * ntn, 8) * 8));
    if (out_fp32)
      hipLaunchKernelGGL(k_gemm_mxfp8_wgrad<true>, grid, dim3(256), 0, st, A, a_scale, B,
                         b_scale, offsets, G, M, N, K, ntm, ntn, out);
    else
      hipLaunchKernelGGL(k_gemm_mxfp8_wgrad<false>, grid, dim3(256), 0, st, A, a_scale, B,
                         b_scale, offsets, G, M, N, K, ntm, ntn, out);
    return hipGetLastError();
  }
  if (fmt == 1 && kind == 1) {  // DGRAD (MXFP8): B = column-wise copy of the stacked weight
    if (M == 0) return hipSuccess;
    if (K % 128 || K / 32 > Mx3<256>::MAX_KS || G * K * 256 + K >= U32)
      return hipErrorNotSupported;
    const uint8_t *A = static_cast<const uint8_t *>(a), *B = static_cast<const uint8_t *>(b);
    const int64_t ntn_b = cdiv(N, Mq<256>::TN);
    if (256 * K < U32 && qp_fits(G, M, N, K, out_fp32 ? 4 : 2)) {
      // the persistent forward kernel with B's row stride G K and expert stride K
      const uint32_t ob = (uint32_t)(M * N * (out_fp32 ? 4 : 2));
      PQM_FB(k_gemm_mxfp8_qp, dim3((unsigned)qp_grid(G, M, N)), dim3(512), A, a_scale, B, b_scale,
             offsets, G, N, K, ntn_b, G * K, K, out, ob, nullptr);
      return hipGetLastError();
    }
    const dim3 grid_b((unsigned)(cdiv((cdiv(M, 256) + G) * ntn_b, 8) * 8));
    if (out_fp32)
      hipLaunchKernelGGL((k_gemm_mxfp8_q<true, false>), grid_b, dim3(512), 0, st, A, a_scale, B,
                         b_scale, offsets, G, N, K, ntn_b, G * K, K, out, nullptr);
    else
      hipLaunchKernelGGL((k_gemm_mxfp8_q<false, false>), grid_b, dim3(512), 0, st, A, a_scale, B,
                         b_scale, offsets, G, N, K, ntn_b, G * K, K, out, nullptr);
    return hipGetLastError();
  }
  if (kind == 2 && K > 0 && M * N * 2 < U32 && M * K * 2 < U32) {  // WGRAD (bf16), pipelined
    const int64_t ntn = cdiv(N, 256), ntk = cdiv(K, 256);
    const dim3 grid((unsigned)(G * ntn * ntk));
    const uint16_t *A = static_cast<const uint16_t *>(a), *B = static_cast<const uint16_t *>(b);
    if (out_fp32)
      hipLaunchKernelGGL((k_gemm_bf16_pipe<BP_WGRAD, true>), grid, dim3(256), 0, st, A, B,
                         offsets, G, N, K, ntn, ntk, out, nullptr);
    else
      hipLaunchKernelGGL((k_gemm_bf16_pipe<BP_WGRAD, false>), grid, dim3(256), 0, st, A, B,
                         offsets, G, N, K, ntn, ntk, out, nullptr);
    return hipGetLastError();
  }
  if (kind == 2) {  // WGRAD (bf16)
    if (K == 0) return hipSuccess;
    const int64_t ntn = cdiv(N, GT_M), ntk = cdiv(K, GT_N);
    const dim3 grid((unsigned)(G * ntn * ntk));
    const uint16_t *A = static_cast<const uint16_t *>(a), *B = static_cast<const uint16_t *>(b);
    if (out_fp32)
      hipLaunchKernelGGL(k_gemm_bf16_wgrad<true>, grid, dim3(256), 0, st, A, B, offsets, N, K,
                         ntn, ntk, out);
    else
      hipLaunchKernelGGL(k_gemm_bf16_wgrad<false>, grid, dim3(256), 0, st, A, B, offsets, N,
                         K, ntn, ntk, out);
    return hipGetLastError();
  }
  if (M == 0) return hipSuccess;
  const int64_t ntn = cdiv(N, GT_N);
  int64_t tiles = (cdiv(M, GT_M) + G) * ntn;
  tiles = cdiv(tiles, 8) * 8;
  const dim3 grid((unsigned)tiles);
  if (fmt == 1 && K > 0 && K % 128 == 0 && 256 * K < U32 &&
      qp_fits(G, M, N, K, out_fp32 ? 4 : 2)) {
    const uint8_t *A = static_cast<const uint8_t *>(a), *B = static_cast<const uint8_t *>(b);
    const int64_t ntn_b = cdiv(N, 256);
    const dim3 grid_p((unsigned)qp_grid(G, M, N));
    const uint32_t ob = (uint32_t)(M * N * (out_fp32 ? 4 : 2));
    PQM_FB(k_gemm_mxfp8_qp, grid_p, dim3(512), A, a_scale, B, b_scale, offsets, G, N, K, ntn_b,
           K, N * K, out, ob, bias);
    return hipGetLastError();
  }
  if (fmt == 1 && K > 0 && K % 128 == 0 && 256 * K < U32) {
    const uint8_t *A = static_cast<const uint8_t *>(a), *B = static_cast<const uint8_t *>(b);
    const int64_t ntn_b = cdiv(N, Mq<256>::TN);
    const dim3 grid_b((unsigned)(cdiv((cdiv(M, 256) + G) * ntn_b, 8) * 8));
    PQM_FB(k_gemm_mxfp8_q, grid_b, dim3(512), A, a_scale, B, b_scale, offsets, G, N, K, ntn_b,
           K, N * K, out, bias);
    return hipGetLastError();
  }
  if (fmt == 1) {
    const uint8_t *A = static_cast<const uint8_t *>(a), *B = static_cast<const uint8_t *>(b);
    if (out_fp32)
      hipLaunchKernelGGL(k_gemm_mxfp8<true>, grid, dim3(256), 0, st, A, a_scale, B, b_scale,
                         offsets, G, N, K, ntn, out, bias);
    else
      hipLaunchKernelGGL(k_gemm_mxfp8<false>, grid, dim3(256), 0, st, A, a_scale, B, b_scale,
                         offsets, G, N, K, ntn, out, bias);
    return hipGetLastError();
  }
  if (fmt == 0 && K % 64 == 0 && (kind == 0 || K * N * 2 < U32)) {
    const uint16_t *A = static_cast<const uint16_t *>(a), *B = static_cast<const uint16_t *>(b);
    const int64_t ntn_b = cdiv(N, 256);
    const dim3 grid_b((unsigned)(cdiv((cdiv(M, 256) + G) * ntn_b, 8) * 8));
    if (kind == 0) {
      if (out_fp32) {
        if (bias)
          hipLaunchKernelGGL((k_gemm_bf16_pipe<BP_FPROP, true, true>), grid_b, dim3(256), 0, st,
                             A, B, offsets, G, N, K, ntn_b, (int64_t)0, out, bias);
        else
          hipLaunchKernelGGL((k_gemm_bf16_pipe<BP_FPROP, true>), grid_b, dim3(256), 0, st, A, B,
                             offsets, G, N, K, ntn_b, (int64_t)0, out, nullptr);
      } else {
        if (bias)
          hipLaunchKernelGGL((k_gemm_bf16_pipe<BP_FPROP, false, true>), grid_b, dim3(256), 0, st,
                             A, B, offsets, G, N, K, ntn_b, (int64_t)0, out, bias);
        else
          hipLaunchKernelGGL((k_gemm_bf16_pipe<BP_FPROP, false>), grid_b, dim3(256), 0, st, A,
                             B, offsets, G, N, K, ntn_b, (int64_t)0, out, nullptr);
      }
    } else {
      if (out_fp32)
        hipLaunchKernelGGL((k_gemm_bf16_pipe<BP_DGRAD, true>), grid_b, dim3(256), 0, st, A, B,
                           offsets, G, N, K, ntn_b, (int64_t)0, out, nullptr);
      else
        hipLaunchKernelGGL((k_gemm_bf16_pipe<BP_DGRAD, false>), grid_b, dim3(256), 0, st, A, B,
                           offsets, G, N, K, ntn_b, (int64_t)0, out, nullptr);
    }
    return hipGetLastError();
  }
  if (fmt == 0) {
    const uint16_t *A = static_cast<const uint16_t *>(a), *B = static_cast<const uint16_t *>(b);
    if (kind == 0) {
      if (out_fp32)
        hipLaunchKernelGGL((k_gemm_bf16_rows<false, true>), grid, dim3(256), 0, st, A, B,
                           offsets, G, N, K, ntn, out, bias);
      else
        hipLaunchKernelGGL((k_gemm_bf16_rows<false, false>), grid, dim3(256), 0, st, A, B,
                           offsets, G, N, K, ntn, out, bias);
    } else {
      if (out_fp32)
        hipLaunchKernelGGL((k_gemm_bf16_rows<true, true>), grid, dim3(256), 0, st, A, B,
                           offsets, G, N, K, ntn, out, nullptr);
      else
        hipLaunchKernelGGL((k_gemm_bf16_rows<true, false>), grid, dim3(256), 0, st, A, B,
                           offsets, G, N, K, ntn, out, nullptr);
    }
    return hipGetLastError();
  }
  if (fmt == 2 && K > 0 && K % 256 == 0 && (uintptr_t)a_scale % 4 == 0 && (uintptr_t)b_scale % 4 == 0 &&
      N >= 512 && M <= 256 * G && !out_fp32 && !bias && npw_fits(G, M, N, K)) {
    // experts of 256 rows or fewer on average, bf16 output: persistent
    const uint8_t *A = static_cast<const uint8_t *>(a), *B = static_cast<const uint8_t *>(b);
    hipLaunchKernelGGL(k_gemm_nvfp4_wide_p, dim3((unsigned)npw_grid(G, M, N)), dim3(256), 0, st, A,
                       a_scale, a_outer, B, b_scale, b_outer, b_rows_per_scale, offsets, G, N, K,
                       cdiv(N, 512), out, (uint32_t)(M * N * 2));
    return hipGetLastError();
  }
  if (fmt == 2 && K > 0 && K % 256 == 0 && (uintptr_t)a_scale % 4 == 0 && (uintptr_t)b_scale % 4 == 0 &&
      N >= 512 && M <= 256 * G) {  // experts of 256 rows or fewer on average
    const uint8_t *A = static_cast<const uint8_t *>(a), *B = static_cast<const uint8_t *>(b);
    const int64_t ntn_w = cdiv(N, 512);
    const dim3 grid_w((unsigned)(cdiv((cdiv(M, 128) + G) * ntn_w, 8) * 8));
    PQM_FB(k_gemm_nvfp4_wide, grid_w, dim3(256), A, a_scale, a_outer, B, b_scale, b_outer,
           b_rows_per_scale, offsets, G, N, K, ntn_w, out, bias);
    return hipGetLastError();
  }
  if (fmt == 2 && K > 0 && K % 256 == 0 && (uintptr_t)a_scale % 4 == 0 && (uintptr_t)b_scale % 4 == 0) {
    const uint8_t *A = static_cast<const uint8_t *>(a), *B = static_cast<const uint8_t *>(b);
    const int64_t ntn_b = cdiv(N, 256);
    const dim3 grid_b((unsigned)(cdiv((cdiv(M, 256) + G) * ntn_b, 8) * 8));
    PQM_FB(k_gemm_nvfp4_pipe, grid_b, dim3(256), A, a_scale, a_outer, B, b_scale, b_outer,
           b_rows_per_scale, offsets, G, N, K, ntn_b, out, bias);
    return hipGetLastError();
  }
  if (fmt == 2) {
    const uint8_t *A = static_cast<const uint8_t *>(a), *B = static_cast<const uint8_t *>(b);
    if (out_fp32)
      hipLaunchKernelGGL(k_gemm_nvfp4<true>, grid, dim3(256), 0, st, A, a_scale, a_outer, B,
                         b_scale, b_outer, b_rows_per_scale, offsets, G, N, K, ntn, out, bias);
    else
      hipLaunchKernelGGL(k_gemm_nvfp4<false>, grid, dim3(256), 0, st, A, a_scale, a_outer, B,
                         b_scale, b_outer, b_rows_per_scale, offsets, G, N, K, ntn, out, bias);
    return hipGetLastError();
  }
#undef PQM_FB
  return hipErrorNotSupported;
}

hipError_t launch_gemm_swiglu_mxfp8(const uint8_t *a, const uint8_t *a_scale, const uint8_t *b,
                                    const uint8_t *b_scale, const int64_t *offsets, int64_t G,
                                    int64_t M, int64_t I, int64_t K, const float *prob,
                                    const int32_t *src, uint8_t *q, uint8_t *s, hipStream_t st) {
  if (G == 0 || M == 0 || I == 0) return hipSuccess;
  const int64_t N = 2 * I, ntn = N / 256;
  if (qp_fits(G, M, N, K, 2) && M * I < (int64_t)QP_OOB) {
    hipLaunchKernelGGL(k_gemm_mxfp8_qp_swiglu, dim3((unsigned)qp_grid(G, M, N)), dim3(512), 0, st,
                       a, a_scale, b, b_scale, offsets, G, N, K, ntn, (uint32_t)(M * I),
                       SwigluEpi{prob, src, I, q, s});
    return hipGetLastError();
  }
  const dim3 grid((unsigned)(cdiv((cdiv(M, 256) + G) * ntn, 8) * 8));
  hipLaunchKernelGGL(k_gemm_mxfp8_swiglu, grid, dim3(256), 0, st, a, a_scale, b, b_scale,
                     offsets, G, N, K, ntn, SwigluEpi{prob, src, I, q, s});
  return hipGetLastError();
}

// Online-amax FC2 (k_gemm_nvfp4_online): K a positive multiple of 256,
// 4-byte aligned W2 block scales (their words are loaded whole).
hipError_t launch_fc2_online_nvfp4(const uint16_t *p, const uint8_t *b, const uint8_t *b_scale,
                                   const float *b_outer, int64_t b_rows_per_scale,
                                   const int64_t *offsets, int64_t G, int64_t M, int64_t N,
                                   int64_t K, void *out, int out_fp32, float *gs_out,
                                   uint8_t *q_out, uint8_t *sb_out, hipStream_t st) {
  if (G == 0 || M == 0 || N == 0) return hipSuccess;
  if (K <= 0 || K % 256 || (uintptr_t)b_scale % 4) return hipErrorNotSupported;
  const int64_t ntn = cdiv(N, NpOn::TN);
  const dim3 grid((unsigned)(cdiv((cdiv(M, NpOn::TMR) + G) * ntn, 8) * 8));
  if (out_fp32)
    hipLaunchKernelGGL(k_gemm_nvfp4_online<true>, grid, dim3(256), 0, st, p, b, b_scale, b_outer,
                       b_rows_per_scale, offsets, G, N, K, ntn, out, gs_out, q_out, sb_out);
  else
    hipLaunchKernelGGL(k_gemm_nvfp4_online<false>, grid, dim3(256), 0, st, p, b, b_scale,
                       b_outer, b_rows_per_scale, offsets, G, N, K, ntn, out, gs_out, q_out,
                       sb_out);
  return hipGetLastError();
}

// Online-amax FC2 split into two kernels (k_online_encode_nvfp4, then
// k_gemm_nvfp4_rescale): K a positive multiple of 256 and at most
// 128 NPO_MAX_NK, 4-byte aligned W2 block scales.
hipError_t launch_fc2_online_nvfp4_split(const uint16_t *p, const uint8_t *b,
                                         const uint8_t *b_scale, const float *b_outer,
                                         int64_t b_rows_per_scale, const int64_t *offsets,
                                         int64_t G, int64_t M, int64_t N, int64_t K, void *out,
                                         int out_fp32, float *gs, uint8_t *q, uint8_t *sb,
                                         float *ratio, hipStream_t st) {
  if (G == 0 || M == 0 || N == 0) return hipSuccess;
  if (K <= 0 || K % 256 || K / 128 > NPO_MAX_NK || (uintptr_t)b_scale % 4)
    return hipErrorNotSupported;
  hipLaunchKernelGGL(k_online_encode_nvfp4, dim3((unsigned)cdiv(M, 32)), dim3(256), 0, st, p,
                     offsets, G, K, q, sb, gs, ratio);
  const int64_t ntn = cdiv(N, NpPipe128::TN);
  const dim3 grid((unsigned)(cdiv((cdiv(M, 128) + G) * ntn, 8) * 8));
  if (out_fp32)
    hipLaunchKernelGGL(k_gemm_nvfp4_rescale<true>, grid, dim3(256), 0, st, q, sb, gs, b, b_scale,
                       b_outer, b_rows_per_scale, offsets, G, N, K, ntn, out, ratio);
  else
    hipLaunchKernelGGL(k_gemm_nvfp4_rescale<false>, grid, dim3(256), 0, st, q, sb, gs, b,
                       b_scale, b_outer, b_rows_per_scale, offsets, G, N, K, ntn, out, ratio);
  return hipGetLastError();
}

}  // namespace pqm
