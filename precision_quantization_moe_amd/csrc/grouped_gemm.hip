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
// the scales go to the matrix core unchanged.  K % 128 == 0 (K <= 3072) runs
// the pipelined 128 x 256 kernel (k_gemm_mxfp8_pipe); other K the simpler
// 128 x 128 kernel with register-staged tiles.  Lane layout (verified on the
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
template <int TN = GT_N>
__device__ bool lookup_row_tile(const int64_t *__restrict__ offsets, int64_t G, int64_t ntn,
                                TileInfo &ti, int64_t *sh) {
  const int lane = threadIdx.x & 63;
  if (threadIdx.x < 64) {
    // pass 1: total row tiles
    int64_t total = 0;
    for (int64_t c0 = 0; c0 < G; c0 += 64) {
      const int64_t g = c0 + lane;
      int64_t cnt = 0;
      if (g < G) cnt = (offsets[g + 1] - offsets[g] + GT_M - 1) / GT_M;
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
          cnt = (hi - lo + GT_M - 1) / GT_M;
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
          row0 = l0 + (mt - base - ex) * GT_M;
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
// optionally scaled in binary32 by alpha_row[row] and alpha_col(col).
template <bool OUT_F32>
__device__ __forceinline__ void store_acc(const v16f &acc, void *out, int64_t ldo, int64_t row0,
                                          int64_t row_end, int64_t n0, int64_t N, int rbase,
                                          int cbase, const float *alpha_row = nullptr,
                                          float alpha_col = 1.0f) {
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
      if (alpha_row) v = (float)((double)v * ((double)alpha_row[row] * (double)alpha_col));
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
    void *__restrict__ out) {
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
                         wn * 64 + 32 * j);
}

// ------------------------------------------------- MXFP8, pipelined large tiles
//
// Workgroup tile 128 rows x 256 columns, one workgroup (4 waves) per CU;
// wave (wm, wn) owns rows 64 wm .. +63 and columns 128 wn .. +127 (2 x 4
// accumulators of 32 x 32 in AGPRs).  Per 64-K step and wave: 12 fragment
// reads (12 KB of LDS) feed 8 MFMAs, and the workgroup moves 24 KB from L2.
//
// Operands reach LDS by direct global->LDS loads (global_load_lds_dwordx4:
// lane l's 16 bytes land at M0 + 16 l), issued from inline assembly so that
// the compiler does not serialise them against the LDS reads of other ring
// slots; the code waits for them explicitly.  The ring has 4 slots of one
// 64-K step each; step k+3 is requested while step k is multiplied; before
// step k a wave waits until only its 12 operations of steps k+1 and k+2 are
// pending and then meets the others at a barrier, which publishes step k and
// frees slot (k+3) % 4 (read during step k-1).  Rows of a slot are 64 bytes
// whose 16-byte chunks are XOR-swizzled by (row / 4) % 4; the swizzle goes
// into the global addresses.  All scale bytes of the tile's rows are loaded
// once, dword-major ([dword][row]), so that 32 lanes reading 32 rows hit 32
// banks.  Rows past the expert's end (A) or past N (B) load a clamped valid
// row; their results are never stored.  Requires K % 128 == 0 and
// K <= 2048 * 4 (the scale area).
namespace mx3 {
constexpr int TN = 256;                           // workgroup tile columns
constexpr int SLOT = (GT_M + TN) * 64;            // 24 KB per ring slot
constexpr int NSLOT = 4;
constexpr int MAX_KS = 96;                        // scale bytes per row (K <= 3072)
constexpr int SCALES = (GT_M + TN) * MAX_KS;      // 36 KB
constexpr int LDS = NSLOT * SLOT + SCALES;        // 132 KB
constexpr int OPS = 6;                            // DMA operations per lane per step
}

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

__device__ __forceinline__ uint32_t lds_addr(const void *p) {
  return (uint32_t)(uintptr_t)p;
}

struct Mx3 {
  const uint8_t *Ab, *Bb;  // tile bases
  uint32_t oa[2], ob[4];   // per-lane sources of the step's chunks (step 0)
  uint32_t ring;           // LDS address of slot 0 (wave-uniform)
  uint32_t wave_off;       // wave * 1024
};

template <int SLOTI>
__device__ __forceinline__ void mx3_issue(const Mx3 &L, int kt) {
  const uint32_t kb = (uint32_t)kt * 64u;
  const uint32_t base = L.ring + SLOTI * mx3::SLOT + L.wave_off;
#pragma unroll
  for (int i = 0; i < 2; ++i)
    dma16(L.Ab + (L.oa[i] + kb), __builtin_amdgcn_readfirstlane(base + i * 4096));
#pragma unroll
  for (int i = 0; i < 4; ++i)
    dma16(L.Bb + (L.ob[i] + kb), __builtin_amdgcn_readfirstlane(base + GT_M * 64 + i * 4096));
}

// Byte offset of 16-byte chunk `chunk` of row `row` in a ring slot.
__device__ __forceinline__ int mx3_off(int row, int chunk) {
  return row * 64 + ((chunk ^ (row >> 2)) & 3) * 16;
}

__device__ __forceinline__ v8i mx3_frag(const uint8_t *tile, int r, int h) {
  const uint4 lo = *reinterpret_cast<const uint4 *>(tile + mx3_off(r, h));
  const uint4 hi = *reinterpret_cast<const uint4 *>(tile + mx3_off(r, 2 + h));
  return v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
}

// Multiply step kt held in slot SLOTI.  Scale byte (row, block b) sits at
// sc[(b / 4) * rows * 4 + row * 4 + b % 4].
template <int SLOTI>
__device__ __forceinline__ void mx3_compute(const uint8_t *lds, int kt, v16f (&acc)[2][4],
                                            int wm, int wn, int lane) {
  const uint8_t *cur = lds + SLOTI * mx3::SLOT;
  const uint8_t *sca = lds + mx3::NSLOT * mx3::SLOT;
  const uint8_t *scb = sca + GT_M * 4;  // B rows follow A rows in each dword plane
  const int h = lane >> 5, r32 = lane & 31;
  const int blk = 2 * kt + h;
  const int plane = (blk >> 2) * (GT_M + mx3::TN) * 4, sub = blk & 3;
  const int sa0 = sca[plane + (wm * 64 + r32) * 4 + sub];
  const int sa1 = sca[plane + (wm * 64 + 32 + r32) * 4 + sub];
  const v8i fa0 = mx3_frag(cur, wm * 64 + r32, h);
  const v8i fa1 = mx3_frag(cur, wm * 64 + 32 + r32, h);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int rb = wn * 128 + 32 * j + r32;
    const v8i fb = mx3_frag(cur + GT_M * 64, rb, h);
    const int sb = scb[plane + rb * 4 + sub];
    acc[0][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fa0, fb, acc[0][j], 0, 0, 0, sa0,
                                                                 0, sb);
    acc[1][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fa1, fb, acc[1][j], 0, 0, 0, sa1,
                                                                 0, sb);
  }
}

template <int SLOTI>
__device__ __forceinline__ void mx3_step(const Mx3 &L, const uint8_t *lds, int kt, int nk,
                                         v16f (&acc)[2][4], int wm, int wn, int lane) {
  // own loads of step kt complete: at most steps kt+1, kt+2 still pending
  if (kt + 2 < nk) vm_wait<2 * mx3::OPS>();
  else if (kt + 1 < nk) vm_wait<mx3::OPS>();
  else vm_wait<0>();
  __builtin_amdgcn_s_barrier();
  if (kt + 3 < nk) mx3_issue<(SLOTI + 3) % 4>(L, kt + 3);
  mx3_compute<SLOTI>(lds, kt, acc, wm, wn, lane);
}

template <bool OUT_F32>
__global__ __launch_bounds__(256, 1) void k_gemm_mxfp8_pipe(
    const uint8_t *__restrict__ A, const uint8_t *__restrict__ As,
    const uint8_t *__restrict__ B, const uint8_t *__restrict__ Bs,
    const int64_t *__restrict__ offsets, int64_t G, int64_t N, int64_t K, int64_t ntn,
    void *__restrict__ out) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[mx3::LDS];
  __shared__ int64_t sh[4];
  TileInfo ti;
  if (!lookup_row_tile<mx3::TN>(offsets, G, ntn, ti, sh)) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const uint32_t KS = (uint32_t)(K / 32), Ku = (uint32_t)K;
  const int rows_a = (int)min(ti.row_end - ti.row0, (int64_t)GT_M);
  const int rows_b = (int)min(N - ti.n0, (int64_t)mx3::TN);
  Mx3 L;
  L.Ab = A + ti.row0 * K;
  L.Bb = B + (ti.g * N + ti.n0) * K;
  L.ring = lds_addr(lds);
  L.wave_off = (uint32_t)wave * 1024u;
  // ring chunk c = 256 i + tid: row c / 4, physical chunk c % 4, which holds
  // logical chunk (c % 4) ^ ((row / 4) % 4)
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int c = tid + 256 * i, r = c >> 2, k = (c & 3) ^ ((r >> 2) & 3);
    L.oa[i] = (uint32_t)min(r, rows_a - 1) * Ku + 16u * k;
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c = tid + 256 * i, r = c >> 2, k = (c & 3) ^ ((r >> 2) & 3);
    L.ob[i] = (uint32_t)min(r, rows_b - 1) * Ku + 16u * k;
  }
  // scale bytes: dword plane p holds dword p of every row (A rows, then B
  // rows); lane t of the p-th pass over 384 rows loads (row, dword p)
  {
    const uint8_t *Asb = As + ti.row0 * (int64_t)KS;
    const uint8_t *Bsb = Bs + (ti.g * N + ti.n0) * (int64_t)KS;
    const uint32_t sbase = lds_addr(lds) + mx3::NSLOT * mx3::SLOT;
    const int nd = (int)(KS / 4);  // dwords per row
    for (int p = 0; p < nd; ++p) {
      // 384 rows per plane: waves 0..3 cover rows 64 w .. +63, then 256 + ...
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const int row = q * 256 + tid;  // 0..511, rows >= 384 unused
        if (q == 1 && wave >= 2) continue;  // rows 384..511 do not exist
        const uint8_t *src = row < GT_M
                                 ? Asb + (int64_t)min(row, rows_a - 1) * KS + 4 * p
                                 : Bsb + (int64_t)min(row - GT_M, rows_b - 1) * KS + 4 * p;
        dma4(src, __builtin_amdgcn_readfirstlane(sbase + (uint32_t)(p * (GT_M + mx3::TN) * 4) +
                                                 (uint32_t)(q * 1024 + wave * 256)));
      }
    }
  }

  v16f acc[2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  const int nk = (int)(K / 64);
  mx3_issue<0>(L, 0);
  if (nk > 1) mx3_issue<1>(L, 1);
  if (nk > 2) mx3_issue<2>(L, 2);
  int kt = 0;
  for (; kt + 4 <= nk; kt += 4) {
    mx3_step<0>(L, lds, kt, nk, acc, wm, wn, lane);
    mx3_step<1>(L, lds, kt + 1, nk, acc, wm, wn, lane);
    mx3_step<2>(L, lds, kt + 2, nk, acc, wm, wn, lane);
    mx3_step<3>(L, lds, kt + 3, nk, acc, wm, wn, lane);
  }
  if (kt < nk) mx3_step<0>(L, lds, kt, nk, acc, wm, wn, lane);
  if (kt + 1 < nk) mx3_step<1>(L, lds, kt + 1, nk, acc, wm, wn, lane);
  if (kt + 2 < nk) mx3_step<2>(L, lds, kt + 2, nk, acc, wm, wn, lane);
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
      store_acc<OUT_F32>(acc[i][j], out, N, ti.row0, ti.row_end, ti.n0, N, wm * 64 + 32 * i,
                         wn * 128 + 32 * j);
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
    void *__restrict__ out) {
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
                         wn * 64 + 32 * j);
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
    void *__restrict__ out) {
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
                         wn * 64 + 32 * j, Ao, ab);
  }
}

// ------------------------------------------------------------------ launch

static int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

hipError_t launch_grouped_gemm(int fmt, int kind, const void *a, const uint8_t *a_scale,
                               const float *a_outer, const void *b, const uint8_t *b_scale,
                               const float *b_outer, int64_t b_rows_per_scale,
                               const int64_t *offsets, int64_t G, int64_t M, int64_t N,
                               int64_t K, void *out, int out_fp32, hipStream_t st) {
  if (G == 0 || N == 0) return hipSuccess;
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
  if (fmt == 1 && K % 128 == 0 && K / 32 <= mx3::MAX_KS) {
    const uint8_t *A = static_cast<const uint8_t *>(a), *B = static_cast<const uint8_t *>(b);
    const int64_t ntn_b = cdiv(N, mx3::TN);
    const dim3 grid_b((unsigned)(cdiv((cdiv(M, GT_M) + G) * ntn_b, 8) * 8));
    if (out_fp32)
      hipLaunchKernelGGL(k_gemm_mxfp8_pipe<true>, grid_b, dim3(256), 0, st, A, a_scale, B,
                         b_scale, offsets, G, N, K, ntn_b, out);
    else
      hipLaunchKernelGGL(k_gemm_mxfp8_pipe<false>, grid_b, dim3(256), 0, st, A, a_scale, B,
                         b_scale, offsets, G, N, K, ntn_b, out);
    return hipGetLastError();
  }
  if (fmt == 1) {
    const uint8_t *A = static_cast<const uint8_t *>(a), *B = static_cast<const uint8_t *>(b);
    if (out_fp32)
      hipLaunchKernelGGL(k_gemm_mxfp8<true>, grid, dim3(256), 0, st, A, a_scale, B, b_scale,
                         offsets, G, N, K, ntn, out);
    else
      hipLaunchKernelGGL(k_gemm_mxfp8<false>, grid, dim3(256), 0, st, A, a_scale, B, b_scale,
                         offsets, G, N, K, ntn, out);
    return hipGetLastError();
  }
  if (fmt == 0) {
    const uint16_t *A = static_cast<const uint16_t *>(a), *B = static_cast<const uint16_t *>(b);
    if (kind == 0) {
      if (out_fp32)
        hipLaunchKernelGGL((k_gemm_bf16_rows<false, true>), grid, dim3(256), 0, st, A, B,
                           offsets, G, N, K, ntn, out);
      else
        hipLaunchKernelGGL((k_gemm_bf16_rows<false, false>), grid, dim3(256), 0, st, A, B,
                           offsets, G, N, K, ntn, out);
    } else {
      if (out_fp32)
        hipLaunchKernelGGL((k_gemm_bf16_rows<true, true>), grid, dim3(256), 0, st, A, B,
                           offsets, G, N, K, ntn, out);
      else
        hipLaunchKernelGGL((k_gemm_bf16_rows<true, false>), grid, dim3(256), 0, st, A, B,
                           offsets, G, N, K, ntn, out);
    }
    return hipGetLastError();
  }
  if (fmt == 2) {
    const uint8_t *A = static_cast<const uint8_t *>(a), *B = static_cast<const uint8_t *>(b);
    if (out_fp32)
      hipLaunchKernelGGL(k_gemm_nvfp4<true>, grid, dim3(256), 0, st, A, a_scale, a_outer, B,
                         b_scale, b_outer, b_rows_per_scale, offsets, G, N, K, ntn, out);
    else
      hipLaunchKernelGGL(k_gemm_nvfp4<false>, grid, dim3(256), 0, st, A, a_scale, a_outer, B,
                         b_scale, b_outer, b_rows_per_scale, offsets, G, N, K, ntn, out);
    return hipGetLastError();
  }
  return hipErrorNotSupported;
}

}  // namespace pqm
