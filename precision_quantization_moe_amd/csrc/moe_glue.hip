// moe_glue.hip -- routing into a contiguous expert-sorted buffer, row
// gather, weighted SwiGLU and combine ("miniTE technical report", 5.2: the
// quantized rows go into one contiguous buffer with offsets for the expert
// boundaries, built on the device; 5.4: D = act(gate, up) x prob; "Towards
// Blackwell-Native 8-bit and 4-bit RL": routed outputs are reduced in high
// precision).
#include "pqm_device.hpp"
#include "pqm_internal.hpp"
#include "pqmoe.h"

#include <map>
#include <mutex>

namespace pqm {

constexpr int ROUTE_CHUNK = 256;  // assignments per workgroup (one per thread)

// Per-chunk histogram of expert ids: counts[chunk * E + e].
__global__ __launch_bounds__(256) void k_route_hist(const int32_t *__restrict__ ids,
                                                    int64_t n, int64_t E,
                                                    int32_t *__restrict__ counts) {
  extern __shared__ int32_t h[];
  for (int64_t e = threadIdx.x; e < E; e += 256) h[e] = 0;
  __syncthreads();
  const int64_t base = (int64_t)blockIdx.x * ROUTE_CHUNK;
  for (int i = threadIdx.x; i < ROUTE_CHUNK; i += 256) {
    const int64_t a = base + i;
    if (a < n) {
      const int32_t e = ids[a];
      if (e >= 0 && e < E) atomicAdd(&h[e], 1);  // ids outside [0, E) are skipped
    }
  }
  __syncthreads();
  for (int64_t e = threadIdx.x; e < E; e += 256) counts[blockIdx.x * E + e] = h[e];
}

// Exclusive prefix of v over the 256 threads of the workgroup (thread
// order) plus `carry`; the 256 values' sum is added to carry.  wsum: 4
// shared slots.  Every thread must call it.
__device__ __forceinline__ int64_t block_excl_scan256(int64_t v, int64_t &carry, int64_t *wsum) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int64_t incl = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int64_t t = __shfl_up(incl, o, 64);
    if (lane >= o) incl += t;
  }
  if (lane == 63) wsum[wave] = incl;
  __syncthreads();
  int64_t before = carry;
  for (int w = 0; w < wave; ++w) before += wsum[w];
  carry += wsum[0] + wsum[1] + wsum[2] + wsum[3];
  __syncthreads();  // every thread has read the slots before they are reused
  return before + incl - v;
}

// One workgroup per expert e: its column of chunk counts becomes, in place,
// the exclusive prefix over chunks (the first row of (chunk, e) relative to
// the expert's first row), and total[e] its sum.
__global__ __launch_bounds__(256) void k_route_colscan(int32_t *__restrict__ counts,
                                                       int64_t nchunks, int64_t E,
                                                       int64_t *__restrict__ total) {
  __shared__ int64_t wsum[4];
  const int64_t e = blockIdx.x;
  int64_t carry = 0;
  for (int64_t c0 = 0; c0 < nchunks; c0 += 256) {
    const int64_t c = c0 + threadIdx.x;
    const int64_t v = c < nchunks ? counts[c * E + e] : 0;
    const int64_t x = block_excl_scan256(v, carry, wsum);
    if (c < nchunks) counts[c * E + e] = (int32_t)x;
  }
  if (threadIdx.x == 0) total[e] = carry;
}

// One workgroup: offsets = exclusive scan of the expert totals (all zero
// when total is NULL).  shared_rows >= 0 (a shared expert, possibly with no
// tokens): offsets[E+1] closes one more group of that many rows after the
// routed ones; -1: no such group.
__global__ __launch_bounds__(256) void k_route_offsets(const int64_t *__restrict__ total,
                                                       int64_t E, int64_t shared_rows,
                                                       int64_t *__restrict__ offsets) {
  __shared__ int64_t wsum[4];
  int64_t carry = 0;
  for (int64_t b = 0; b < E; b += 256) {
    const int64_t e = b + threadIdx.x;
    const int64_t x = block_excl_scan256(e < E && total ? total[e] : 0, carry, wsum);
    if (e < E) offsets[e] = x;
  }
  if (threadIdx.x == 0) {
    offsets[E] = carry;
    if (shared_rows >= 0) offsets[E + 1] = carry + shared_rows;
  }
}

// Scatter each chunk in flat order: position = start of (chunk, expert) +
// number of earlier assignments of the same expert in the chunk.
__global__ __launch_bounds__(256) void k_route_scatter(const int32_t *__restrict__ ids,
                                                       int64_t n, int64_t E, int64_t k,
                                                       const int32_t *__restrict__ start,
                                                       const int64_t *__restrict__ offsets,
                                                       int32_t *__restrict__ src_row,
                                                       int32_t *__restrict__ token,
                                                       int32_t *__restrict__ slot) {
  extern __shared__ int32_t sh[];
  int32_t *run = sh;          // [E]
  int32_t *round_ids = sh + E;  // [256]
  for (int64_t e = threadIdx.x; e < E; e += 256)
    run[e] = start[blockIdx.x * E + e] + (int32_t)offsets[e];
  const int64_t base = (int64_t)blockIdx.x * ROUTE_CHUNK;
  for (int r = 0; r < ROUTE_CHUNK / 256; ++r) {
    const int64_t a = base + r * 256 + threadIdx.x;
    int32_t e = a < n ? ids[a] : -1;
    if (e >= E) e = -1;
    round_ids[threadIdx.x] = e;
    __syncthreads();
    if (e >= 0) {
      int32_t rank = 0;
      for (int j = 0; j < (int)threadIdx.x; ++j) rank += (round_ids[j] == e) ? 1 : 0;
      const int32_t pos = run[e] + rank;
      src_row[pos] = (int32_t)a;
      token[pos] = (int32_t)(a / k);
      slot[a] = pos;
    }
    __syncthreads();
    if (e >= 0) atomicAdd(&run[e], 1);
    __syncthreads();
  }
}

// Workspace: the (chunk, expert) counts as int32, then the expert totals as
// int64 (8-byte aligned).
static int64_t route_totals_offset(int64_t nchunks, int64_t E) {
  return (nchunks * E * (int64_t)sizeof(int32_t) + 7) / 8 * 8;
}

size_t route_workspace_bytes(int64_t T, int64_t k, int64_t E) {
  const int64_t n = T * k;
  const int64_t nchunks = (n + ROUTE_CHUNK - 1) / ROUTE_CHUNK;
  if (nchunks == 0) return 0;  // no assignments: the offsets are all zero
  return (size_t)(route_totals_offset(nchunks, E) + E * (int64_t)sizeof(int64_t));
}

// The shared expert's rows: row n + t is token t (assignment index n + t).
__global__ void k_route_shared(int64_t n, int64_t T, int32_t *__restrict__ src_row,
                               int32_t *__restrict__ token) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t < T) {
    src_row[n + t] = (int32_t)(n + t);
    token[n + t] = (int32_t)t;
  }
}

hipError_t launch_route(const int32_t *ids, int64_t T, int64_t k, int64_t E, int shared,
                        int64_t *offsets, int32_t *src_row, int32_t *token, int32_t *slot,
                        void *ws, hipStream_t st) {
  const int64_t n = T * k;
  const int64_t nchunks = (n + ROUTE_CHUNK - 1) / ROUTE_CHUNK;
  // with no assignments the workspace may be absent: no counts, and the
  // offsets come from zero totals (total == NULL)
  int32_t *counts = static_cast<int32_t *>(ws);
  int64_t *total = nchunks > 0 ? reinterpret_cast<int64_t *>(static_cast<uint8_t *>(ws) +
                                                             route_totals_offset(nchunks, E))
                               : nullptr;
  if (nchunks > 0) {
    hipLaunchKernelGGL(k_route_hist, dim3((unsigned)nchunks), dim3(256), E * sizeof(int32_t),
                       st, ids, n, E, counts);
    hipLaunchKernelGGL(k_route_colscan, dim3((unsigned)E), dim3(256), 0, st, counts, nchunks, E,
                       total);
  }
  hipLaunchKernelGGL(k_route_offsets, dim3(1), dim3(256), 0, st, total, E,
                     shared ? T : (int64_t)-1, offsets);
  if (nchunks > 0)
    hipLaunchKernelGGL(k_route_scatter, dim3((unsigned)nchunks), dim3(256),
                       (E + 256) * sizeof(int32_t), st, ids, n, E, k, counts, offsets, src_row,
                       token, slot);
  if (shared && T > 0)
    hipLaunchKernelGGL(k_route_shared, dim3((unsigned)((T + 255) / 256)), dim3(256), 0, st, n,
                       T, src_row, token);
  return hipGetLastError();
}

// Routing scratch for callers that cannot allocate (pqm_moe_route_noalloc):
// one file-scope device array per GPU, holding the (chunk, expert) counts
// and the expert totals exactly as the caller workspace of pqm_moe_route
// does.  Every entry is written before it is read, so nothing is cleared
// between calls.  In host code `route_scratch` names a host-side stand-in,
// not device memory: kernels get the per-device address that
// hipGetSymbolAddress returns (route_scratch_ptr).
static __device__ __align__(256) uint8_t route_scratch[PQM_ROUTE_NOALLOC_SCRATCH_BYTES];

// The device address of this device's route_scratch, looked up once per
// device with that device current; NULL if the lookup failed.
static void *route_scratch_ptr() {
  static std::mutex mu;
  static std::map<int, void *> addr;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return nullptr;
  std::lock_guard<std::mutex> lock(mu);
  auto it = addr.find(dev);
  if (it != addr.end()) return it->second;
  void *p = nullptr;
  if (hipGetSymbolAddress(&p, HIP_SYMBOL(route_scratch)) != hipSuccess) p = nullptr;
  if (p) addr[dev] = p;
  return p;
}

// out[i] = src[index[i] / divisor], rows of row_bytes bytes.
template <typename V>
__global__ __launch_bounds__(256) void k_gather(const uint8_t *__restrict__ src,
                                                int64_t row_bytes,
                                                const int32_t *__restrict__ index, int64_t n,
                                                int64_t divisor, uint8_t *__restrict__ out) {
  const int64_t per_row = row_bytes / sizeof(V);
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n * per_row) return;
  const int64_t r = i / per_row, c = i % per_row;
  const int64_t s = index[r] / divisor;
  reinterpret_cast<V *>(out + r * row_bytes)[c] =
      reinterpret_cast<const V *>(src + s * row_bytes)[c];
}

hipError_t launch_gather(const void *src, int64_t row_bytes, const int32_t *index, int64_t n,
                         int64_t divisor, void *out, hipStream_t st) {
  if (n == 0 || row_bytes == 0) return hipSuccess;
  const uint8_t *s = static_cast<const uint8_t *>(src);
  uint8_t *o = static_cast<uint8_t *>(out);
  const bool a16 = row_bytes % 16 == 0 && (uintptr_t)s % 16 == 0 && (uintptr_t)o % 16 == 0;
  const bool a4 = row_bytes % 4 == 0 && (uintptr_t)s % 4 == 0 && (uintptr_t)o % 4 == 0;
  if (a16) {
    const int64_t tot = n * (row_bytes / 16);
    hipLaunchKernelGGL(k_gather<uint4>, dim3((unsigned)((tot + 255) / 256)), dim3(256), 0, st,
                       s, row_bytes, index, n, divisor, o);
  } else if (a4) {
    const int64_t tot = n * (row_bytes / 4);
    hipLaunchKernelGGL(k_gather<uint32_t>, dim3((unsigned)((tot + 255) / 256)), dim3(256), 0,
                       st, s, row_bytes, index, n, divisor, o);
  } else {
    const int64_t tot = n * row_bytes;
    hipLaunchKernelGGL(k_gather<uint8_t>, dim3((unsigned)((tot + 255) / 256)), dim3(256), 0,
                       st, s, row_bytes, index, n, divisor, o);
  }
  return hipGetLastError();
}

// Eight outputs d[m, j .. j+7] = bf16( silu(g) * u * p ), g = c[m, j..],
// u = c[m, I + j..], p = the router probability of the assignment stored at
// row m, as 4 words of bf16 pairs.
__device__ __forceinline__ void swiglu8(const uint16_t *__restrict__ c,
                                        const float *__restrict__ prob,
                                        const int32_t *__restrict__ src, int64_t I, int64_t m,
                                        int64_t j, uint32_t (&o)[4]) {
  const float p = prob[src ? src[m] : m];
  const uint4 gv = *reinterpret_cast<const uint4 *>(c + m * 2 * I + j);
  const uint4 uv = *reinterpret_cast<const uint4 *>(c + m * 2 * I + I + j);
  const uint32_t gw[4] = {gv.x, gv.y, gv.z, gv.w}, uw[4] = {uv.x, uv.y, uv.z, uv.w};
#pragma unroll
  for (int k = 0; k < 4; ++k)
    o[k] = pk_bf16_rne(swiglu_f32(bf16_lo_f32(gw[k]), bf16_lo_f32(uw[k]), p),
                       swiglu_f32(bf16_hi_f32(gw[k]), bf16_hi_f32(uw[k]), p));
}

// d = swiglu8 per lane (16-byte bf16 loads and stores).
__global__ __launch_bounds__(256) void k_swiglu_prob(const uint16_t *__restrict__ c,
                                                     const float *__restrict__ prob,
                                                     const int32_t *__restrict__ src,
                                                     int64_t M, int64_t I,
                                                     uint16_t *__restrict__ d) {
  const int64_t per_row = I / 8;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= M * per_row) return;
  const int64_t m = i / per_row, j = (i % per_row) * 8;
  uint32_t o[4];
  swiglu8(c, prob, src, I, m, j, o);
  *reinterpret_cast<uint4 *>(d + m * I + j) = make_uint4(o[0], o[1], o[2], o[3]);
}

// The same d, quantized in place to MXFP8 row-wise (1 x 32 blocks along j):
// the 4 lanes of a block (consecutive lanes, I % 32 == 0) reduce its
// maximum with two quad permutes; the E8M0 byte and the E4M3 codes follow
// the quantizer's rules, so q and s equal pqm_quantize_mxfp8 of d.  d is
// written too when non-null.
__global__ __launch_bounds__(256) void k_swiglu_quant_mxfp8(
    const uint16_t *__restrict__ c, const float *__restrict__ prob,
    const int32_t *__restrict__ src, int64_t M, int64_t I, uint16_t *__restrict__ d,
    uint8_t *__restrict__ q, uint8_t *__restrict__ s) {
  const int64_t per_row = I / 8;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= M * per_row) return;  // whole quads: M * per_row is a multiple of 4
  const int64_t m = i / per_row, j = (i % per_row) * 8;
  uint32_t o[4];
  swiglu8(c, prob, src, I, m, j, o);
  if (d) *reinterpret_cast<uint4 *>(d + m * I + j) = make_uint4(o[0], o[1], o[2], o[3]);
  uint32_t mm = pk_max_u16(pk_max_u16(o[0] & 0x7FFF7FFFu, o[1] & 0x7FFF7FFFu),
                           pk_max_u16(o[2] & 0x7FFF7FFFu, o[3] & 0x7FFF7FFFu));
  mm = max(mm & 0xFFFFu, mm >> 16);
  mm = max(mm, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)mm, 0xB1, 0xF, 0xF, false));
  mm = max(mm, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)mm, 0x4E, 0xF, 0xF, false));
  const uint32_t b = mx_scale_byte(mm);
  const float scale = __uint_as_float(b << 23);  // the E8M0 byte as the conversion's scale
  *reinterpret_cast<uint2 *>(q + m * I + j) =
      make_uint2(cvt4_e4m3_bf16(o[0], o[1], scale), cvt4_e4m3_bf16(o[2], o[3], scale));
  if ((threadIdx.x & 3) == 0) s[m * (I / 32) + j / 32] = (uint8_t)b;
}

hipError_t launch_swiglu_quant_mxfp8(const uint16_t *c, const float *prob, const int32_t *src,
                                     int64_t M, int64_t I, uint16_t *d, uint8_t *q, uint8_t *s,
                                     hipStream_t st) {
  const int64_t tot = M * (I / 8);
  if (tot == 0) return hipSuccess;
  hipLaunchKernelGGL(k_swiglu_quant_mxfp8, dim3((unsigned)((tot + 255) / 256)), dim3(256), 0, st,
                     c, prob, src, M, I, d, q, s);
  return hipGetLastError();
}

hipError_t launch_swiglu(const uint16_t *c, const float *prob, const int32_t *src, int64_t M,
                         int64_t I, uint16_t *d, hipStream_t st) {
  const int64_t tot = M * (I / 8);
  if (tot == 0) return hipSuccess;
  hipLaunchKernelGGL(k_swiglu_prob, dim3((unsigned)((tot + 255) / 256)), dim3(256), 0, st, c,
                     prob, src, M, I, d);
  return hipGetLastError();
}

// out[t, n] = bf16( sum_j y[slot[t, j], n] (+ shared[t, n]) ), summed in
// binary32 in j order.
__global__ __launch_bounds__(256) void k_combine(const uint16_t *__restrict__ y,
                                                 const int32_t *__restrict__ slot,
                                                 const uint16_t *__restrict__ shared,
                                                 int64_t T, int64_t k, int64_t N,
                                                 uint16_t *__restrict__ out) {
  const int64_t per_row = N / 8;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= T * per_row) return;
  const int64_t t = i / per_row, n = (i % per_row) * 8;
  float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  // batches of 8 slots: all index loads, then all row loads in flight
  // together, then the sums in j order
  constexpr int KB = 8;
  for (int64_t j0 = 0; j0 < k; j0 += KB) {
    int64_t r[KB];
    uint4 v[KB];
#pragma unroll
    for (int u = 0; u < KB; ++u) r[u] = j0 + u < k ? (int64_t)slot[t * k + j0 + u] : -1;
#pragma unroll
    for (int u = 0; u < KB; ++u)
      v[u] = r[u] >= 0 ? *reinterpret_cast<const uint4 *>(y + r[u] * N + n) : make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int u = 0; u < KB; ++u) {
      if (r[u] < 0) break;
      const uint32_t w[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        acc[2 * q] += bf16_lo_f32(w[q]);
        acc[2 * q + 1] += bf16_hi_f32(w[q]);
      }
    }
  }
  if (shared) {
    const uint4 v = *reinterpret_cast<const uint4 *>(shared + t * N + n);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      acc[2 * q] += bf16_lo_f32(w[q]);
      acc[2 * q + 1] += bf16_hi_f32(w[q]);
    }
  }
  *reinterpret_cast<uint4 *>(out + t * N + n) =
      make_uint4(pk_bf16_rne(acc[0], acc[1]), pk_bf16_rne(acc[2], acc[3]),
                 pk_bf16_rne(acc[4], acc[5]), pk_bf16_rne(acc[6], acc[7]));
}

hipError_t launch_combine(const uint16_t *y, const int32_t *slot, const uint16_t *shared,
                          int64_t T, int64_t k, int64_t N, uint16_t *out, hipStream_t st) {
  const int64_t tot = T * (N / 8);
  if (tot == 0) return hipSuccess;
  hipLaunchKernelGGL(k_combine, dim3((unsigned)((tot + 255) / 256)), dim3(256), 0, st, y, slot,
                     shared, T, k, N, out);
  return hipGetLastError();
}

// Per-expert padding to whole blocks of `align` rows, so that column-wise
// (32 x 1) blocks never hold two experts' tokens.  One workgroup scans the
// padded counts: poff[g] = sum over e < g of ceil(n_e / align) * align.
__global__ __launch_bounds__(1024) void k_pad_offsets(const int64_t *__restrict__ off, int64_t G,
                                                      int64_t align, int64_t *__restrict__ poff) {
  __shared__ int64_t part[1024];
  int64_t carry = 0;
  for (int64_t c0 = 0; c0 < G; c0 += 1024) {
    const int64_t g = c0 + threadIdx.x;
    int64_t v = 0;
    if (g < G) v = (off[g + 1] - off[g] + align - 1) / align * align;
    part[threadIdx.x] = v;
    __syncthreads();
    for (int o = 1; o < 1024; o <<= 1) {  // inclusive scan
      const int64_t t = threadIdx.x >= o ? part[threadIdx.x - o] : 0;
      __syncthreads();
      part[threadIdx.x] += t;
      __syncthreads();
    }
    if (g < G) poff[g + 1] = carry + part[threadIdx.x];
    carry += part[1023];
    __syncthreads();
  }
  if (threadIdx.x == 0) poff[0] = 0;
}

// One wave per output row: find its group in poff (binary search), then
// copy the source row or write zeros, 16 bytes per lane.
__global__ __launch_bounds__(256) void k_pad_rows(const uint8_t *__restrict__ src,
                                                  int64_t row_bytes,
                                                  const int64_t *__restrict__ off,
                                                  const int64_t *__restrict__ poff, int64_t G,
                                                  uint8_t *__restrict__ out, int64_t out_rows) {
  const int lane = threadIdx.x & 63;
  const int64_t p = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (p >= out_rows) return;
  int64_t srow = -1;
  if (p < poff[G]) {
    int64_t lo = 0, hi = G;  // largest g with poff[g] <= p
    while (hi - lo > 1) {
      const int64_t mid = (lo + hi) / 2;
      if (poff[mid] <= p) lo = mid; else hi = mid;
    }
    const int64_t j = p - poff[lo];
    if (j < off[lo + 1] - off[lo]) srow = off[lo] + j;
  }
  uint4 *o = reinterpret_cast<uint4 *>(out + p * row_bytes);
  const int64_t nv = row_bytes / 16;
  if (srow >= 0) {
    const uint4 *s = reinterpret_cast<const uint4 *>(src + srow * row_bytes);
    for (int64_t c = lane; c < nv; c += 64) o[c] = s[c];
  } else {
    for (int64_t c = lane; c < nv; c += 64) o[c] = make_uint4(0, 0, 0, 0);
  }
}

hipError_t launch_pad_rows(const void *src, int64_t row_bytes, const int64_t *off, int64_t G,
                           int64_t align, int64_t *poff, void *out, int64_t out_rows,
                           hipStream_t st) {
  hipLaunchKernelGGL(k_pad_offsets, dim3(1), dim3(1024), 0, st, off, G, align, poff);
  if (out_rows > 0 && row_bytes > 0)
    hipLaunchKernelGGL(k_pad_rows, dim3((unsigned)((out_rows + 3) / 4)), dim3(256), 0, st,
                       static_cast<const uint8_t *>(src), row_bytes, off, poff, G,
                       static_cast<uint8_t *>(out), out_rows);
  return hipGetLastError();
}

// Offsets check for callers that want one (the GEMMs take the offsets on
// trust): scan i = 0 .. G and report the first index that breaks the
// contract, with the first check it breaks at that index.  One workgroup;
// each thread keeps its first failure, then a block minimum.
__global__ __launch_bounds__(1024) void k_validate_offsets(const int64_t *__restrict__ off,
                                                            int64_t G, int64_t M_total,
                                                            int64_t align,
                                                            int32_t *__restrict__ result) {
  __shared__ int64_t best[1024];
  int64_t mine = INT64_MAX;  // (index << 3) | code of this thread's first failure
  for (int64_t i = threadIdx.x; i <= G; i += blockDim.x) {
    const int64_t v = off[i];
    int code = 0;
    if (i == 0 && v != 0) code = PQM_OFFSETS_FIRST_NOT_ZERO;
    else if (i < G && off[i + 1] < v) code = PQM_OFFSETS_DECREASING;
    else if (v % align != 0) code = PQM_OFFSETS_MISALIGNED;
    else if (i == G && v > M_total) code = PQM_OFFSETS_PAST_END;
    if (code) {
      mine = (i << 3) | code;
      break;  // later indices of this thread are larger
    }
  }
  best[threadIdx.x] = mine;
  __syncthreads();
  for (int w = blockDim.x / 2; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) best[threadIdx.x] = min(best[threadIdx.x], best[threadIdx.x + w]);
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    const int64_t b = best[0];
    result[0] = b == INT64_MAX ? 0 : (int32_t)(b & 7);
    result[1] = b == INT64_MAX ? -1 : (int32_t)min(b >> 3, (int64_t)INT32_MAX);
  }
}

hipError_t launch_validate_offsets(const int64_t *off, int64_t G, int64_t M_total, int64_t align,
                                   int32_t *result, hipStream_t st) {
  hipLaunchKernelGGL(k_validate_offsets, dim3(1), dim3(1024), 0, st, off, G, M_total, align,
                     result);
  return hipGetLastError();
}

}  // namespace pqm

namespace {
bool al(const void *p, size_t a) { return ((uintptr_t)p % a) == 0; }
pqm_status st_of(hipError_t e) { return e == hipSuccess ? PQM_OK : PQM_ERR_HIP; }
}  // namespace

extern "C" {

size_t pqm_moe_route_workspace(int64_t tokens, int64_t k, int64_t num_experts) {
  if (tokens <= 0 || k <= 0 || num_experts <= 0) return 0;
  return pqm::route_workspace_bytes(tokens, k, num_experts);
}

pqm_status pqm_moe_route(const int32_t *topk_ids, int64_t tokens, int64_t k,
                         int64_t num_experts, int shared_expert, int64_t *offsets,
                         int32_t *src_row, int32_t *token, int32_t *slot, void *workspace,
                         size_t workspace_bytes, hipStream_t stream) {
  if (tokens < 0 || k < 1 || num_experts < 1 || num_experts > 4096) return PQM_ERR_SHAPE;
  if (tokens * (k + 1) > (int64_t)0x7FFFFFFF) return PQM_ERR_SHAPE;
  if (!offsets) return PQM_ERR_NULL;
  if (shared_expert != 0 && shared_expert != 1) return PQM_ERR_ENUM;
  if (tokens > 0 && (!topk_ids || !src_row || !token || !slot || !workspace))
    return PQM_ERR_NULL;
  if (workspace_bytes < pqm::route_workspace_bytes(tokens, k, num_experts))
    return PQM_ERR_WORKSPACE;
  if (!al(offsets, 8) || (workspace && !al(workspace, 8))) return PQM_ERR_ALIGN;
  return st_of(pqm::launch_route(topk_ids, tokens, k, num_experts, shared_expert, offsets,
                                 src_row, token, slot, workspace, stream));
}

pqm_status pqm_moe_route_noalloc(const int32_t *topk_ids, int64_t tokens, int64_t k,
                                 int64_t num_experts, int shared_expert, int64_t *offsets,
                                 int32_t *src_row, int32_t *token, int32_t *slot,
                                 hipStream_t stream) {
  if (tokens < 0 || k < 1 || num_experts < 1 || num_experts > 4096) return PQM_ERR_SHAPE;
  if (tokens * (k + 1) > (int64_t)0x7FFFFFFF) return PQM_ERR_SHAPE;
  if (!offsets) return PQM_ERR_NULL;
  if (shared_expert != 0 && shared_expert != 1) return PQM_ERR_ENUM;
  if (tokens > 0 && (!topk_ids || !src_row || !token || !slot)) return PQM_ERR_NULL;
  if (pqm::route_workspace_bytes(tokens, k, num_experts) > PQM_ROUTE_NOALLOC_SCRATCH_BYTES)
    return PQM_ERR_WORKSPACE;
  if (!al(offsets, 8)) return PQM_ERR_ALIGN;
  void *ws = nullptr;
  if (pqm::route_workspace_bytes(tokens, k, num_experts) > 0) {
    ws = pqm::route_scratch_ptr();
    if (!ws) return PQM_ERR_HIP;
  }
  return st_of(pqm::launch_route(topk_ids, tokens, k, num_experts, shared_expert, offsets,
                                 src_row, token, slot, ws, stream));
}

pqm_status pqm_moe_gather_rows(const void *src, int64_t src_rows, int64_t row_bytes,
                               const int32_t *index, int64_t n, int64_t divisor, void *out,
                               hipStream_t stream) {
  (void)src_rows;
  if (src_rows < 0 || row_bytes < 0 || n < 0 || divisor < 1) return PQM_ERR_SHAPE;
  if (n == 0 || row_bytes == 0) return PQM_OK;
  if (!src || !index || !out) return PQM_ERR_NULL;
  return st_of(pqm::launch_gather(src, row_bytes, index, n, divisor, out, stream));
}

pqm_status pqm_moe_pad_rows(const void *src, int64_t src_rows, int64_t row_bytes,
                            const int64_t *offsets, int64_t G, int64_t align,
                            int64_t *padded_offsets, void *out, int64_t out_rows,
                            hipStream_t stream) {
  if (src_rows < 0 || row_bytes < 0 || G < 0 || align < 1 || out_rows < 0) return PQM_ERR_SHAPE;
  if (row_bytes % 16 || out_rows < src_rows + G * (align - 1) || out_rows >= ((int64_t)1 << 40))
    return PQM_ERR_SHAPE;
  if (!offsets || !padded_offsets) return PQM_ERR_NULL;
  if (out_rows > 0 && row_bytes > 0 && (!out || (src_rows > 0 && !src))) return PQM_ERR_NULL;
  if (!al(offsets, 8) || !al(padded_offsets, 8) || !al(src, 16) || !al(out, 16))
    return PQM_ERR_ALIGN;
  return st_of(pqm::launch_pad_rows(src, row_bytes, offsets, G, align, padded_offsets, out,
                                    out_rows, stream));
}

pqm_status pqm_swiglu_prob(const uint16_t *c, const float *prob, const int32_t *src,
                           int64_t rows, int64_t inter, uint16_t *d, hipStream_t stream) {
  if (rows < 0 || inter < 0 || inter % 8) return PQM_ERR_SHAPE;
  if (rows == 0 || inter == 0) return PQM_OK;
  if (!c || !prob || !d) return PQM_ERR_NULL;
  if (!al(c, 16) || !al(d, 16)) return PQM_ERR_ALIGN;
  return st_of(pqm::launch_swiglu(c, prob, src, rows, inter, d, stream));
}

pqm_status pqm_swiglu_prob_quantize_mxfp8(const uint16_t *c, const float *prob,
                                          const int32_t *src, int64_t rows, int64_t inter,
                                          uint16_t *d, uint8_t *q, uint8_t *s,
                                          hipStream_t stream) {
  if (rows < 0 || inter < 0 || inter % 32) return PQM_ERR_SHAPE;
  if (rows == 0 || inter == 0) return PQM_OK;
  if (!c || !prob || !q || !s) return PQM_ERR_NULL;
  if (!al(c, 16) || (d && !al(d, 16)) || !al(q, 8)) return PQM_ERR_ALIGN;
  return st_of(pqm::launch_swiglu_quant_mxfp8(c, prob, src, rows, inter, d, q, s, stream));
}

pqm_status pqm_swiglu_prob_quantize_nvfp4(const uint16_t *c, const float *prob,
                                          const int32_t *src, int64_t rows, int64_t inter,
                                          uint16_t *d, uint8_t *q, uint8_t *s_block,
                                          float *s_outer, hipStream_t stream) {
  if (rows < 0 || inter < 0 || inter % 16 || inter > pqm::nvfp4_max_cols() ||
      rows >= ((int64_t)1 << 31))
    return PQM_ERR_SHAPE;
  if (rows == 0 || inter == 0) return PQM_OK;
  if (!c || !prob || !q || !s_block || !s_outer) return PQM_ERR_NULL;
  if (!al(c, 16) || !al(q, 8) || !al(s_outer, 4) || (d && !al(d, 16))) return PQM_ERR_ALIGN;
  return st_of(pqm::launch_swiglu_quant_nvfp4(c, prob, src, rows, inter, d, q, s_block, s_outer,
                                               stream));
}

pqm_status pqm_moe_combine(const uint16_t *y_rows, const int32_t *slot, const uint16_t *shared,
                           int64_t tokens, int64_t k, int64_t N, uint16_t *out,
                           hipStream_t stream) {
  if (tokens < 0 || k < 1 || N < 0 || N % 8) return PQM_ERR_SHAPE;
  if (tokens == 0 || N == 0) return PQM_OK;
  if (!y_rows || !slot || !out) return PQM_ERR_NULL;
  if (!al(y_rows, 16) || !al(out, 16) || (shared && !al(shared, 16))) return PQM_ERR_ALIGN;
  return st_of(pqm::launch_combine(y_rows, slot, shared, tokens, k, N, out, stream));
}

pqm_status pqm_validate_offsets(const int64_t *offsets, int64_t G, int64_t M_total, int64_t align,
                                int32_t *result, hipStream_t stream) {
  if (G < 0 || M_total < 0 || align < 1) return PQM_ERR_SHAPE;
  if (!offsets || !result) return PQM_ERR_NULL;
  if (!al(offsets, 8) || !al(result, 4)) return PQM_ERR_ALIGN;
  return st_of(pqm::launch_validate_offsets(offsets, G, M_total, align, result, stream));
}

}  // extern "C"
