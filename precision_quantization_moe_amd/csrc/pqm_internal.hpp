// pqm_internal.hpp -- launchers shared between the kernel files and the
// C-ABI layer (not part of the public interface).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace pqm {

// Number of workgroups of `kernel` (block threads, dynamic LDS bytes) that
// can be resident on the current device at once: occupancy per CU times
// the CU count.  Cached per (kernel, device); host-only queries.
int64_t resident_workgroups(const void *kernel, int block, size_t dyn_lds);

// Persistent grid size: min(work items, resident workgroups).
inline unsigned persistent_grid(const void *kernel, int block, size_t dyn_lds, int64_t work) {
  const int64_t r = resident_workgroups(kernel, block, dyn_lds);
  return (unsigned)(work < r ? (work > 0 ? work : 1) : r);
}

hipError_t launch_quantize_mxfp8(const uint16_t *x, int64_t R, int64_t C, int64_t ld,
                                 uint8_t *q, uint8_t *s, uint8_t *qT, uint8_t *sT,
                                 hipStream_t st);

hipError_t launch_quantize_nvfp4(const uint16_t *x, int64_t R, int64_t C, int64_t ld,
                                 int64_t rows_per_scale, uint8_t *q, uint8_t *sb, float *sg,
                                 void *workspace, hipStream_t st);
size_t nvfp4_workspace_bytes(int64_t R, int64_t rows_per_scale);
hipError_t launch_swiglu_quant_nvfp4(const uint16_t *c, const float *prob, const int32_t *src,
                                     int64_t M, int64_t I, uint16_t *d, uint8_t *q, uint8_t *sb,
                                     float *sg, hipStream_t st);
int64_t nvfp4_max_cols();

hipError_t launch_dequantize(int fmt, const uint8_t *q, const uint8_t *s, const float *sg,
                             int64_t R, int64_t C, int64_t rows_per_scale, uint16_t *y,
                             hipStream_t st);

hipError_t launch_gemm_swiglu_mxfp8(const uint8_t *a, const uint8_t *a_scale, const uint8_t *b,
                                    const uint8_t *b_scale, const int64_t *offsets, int64_t G,
                                    int64_t M, int64_t I, int64_t K, const float *prob,
                                    const int32_t *src, uint8_t *q, uint8_t *s, hipStream_t st);
hipError_t launch_quantize_fp8_block(const uint16_t *x, int64_t R, int64_t C, int64_t ld,
                                     int64_t br, uint8_t *q, float *s, hipStream_t st);
hipError_t launch_pad_rows(const void *src, int64_t row_bytes, const int64_t *off, int64_t G,
                           int64_t align, int64_t *poff, void *out, int64_t out_rows,
                           hipStream_t st);
hipError_t launch_grouped_gemm(int fmt, int kind, const void *a, const uint8_t *a_scale,
                               const float *a_outer, const void *b, const uint8_t *b_scale,
                               const float *b_outer, int64_t b_rows_per_scale,
                               const int64_t *offsets, int64_t G, int64_t M, int64_t N,
                               int64_t K, void *out, int out_fp32, const float *bias,
                               uint32_t *ctr, hipStream_t st);
// Workspace bytes the grouped GEMM uses for (fmt, kind): a tile counter for
// the MXFP8 weight gradient, none otherwise.
int64_t grouped_gemm_workspace_bytes(int fmt, int kind);
hipError_t launch_fc2_online_nvfp4(const uint16_t *p, const uint8_t *b, const uint8_t *b_scale,
                                   const float *b_outer, int64_t b_rows_per_scale,
                                   const int64_t *offsets, int64_t G, int64_t M, int64_t N,
                                   int64_t K, void *out, int out_fp32, float *gs_out,
                                   uint8_t *q_out, uint8_t *sb_out, hipStream_t st);
hipError_t launch_fc2_online_nvfp4_split(const uint16_t *p, const uint8_t *b,
                                         const uint8_t *b_scale, const float *b_outer,
                                         int64_t b_rows_per_scale, const int64_t *offsets,
                                         int64_t G, int64_t M, int64_t N, int64_t K, void *out,
                                         int out_fp32, float *gs, uint8_t *q, uint8_t *sb,
                                         float *ratio, hipStream_t st);
hipError_t launch_validate_offsets(const int64_t *off, int64_t G, int64_t M_total, int64_t align,
                                   int32_t *result, hipStream_t st);

}  // namespace pqm
