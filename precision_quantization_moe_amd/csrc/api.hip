// api.hip -- the C ABI declared in include/pqmoe.h: host-side argument
// validation (synchronous, nothing is enqueued on error) and dispatch to the
// kernel launchers.
#include "pqmoe.h"
#include "pqm_internal.hpp"

#include <mutex>
#include <map>
#include <utility>

namespace pqm {

int64_t resident_workgroups(const void *kernel, int block, size_t dyn_lds) {
  static std::mutex mu;
  static std::map<std::pair<const void *, int>, int64_t> cache;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) dev = 0;
  std::lock_guard<std::mutex> lock(mu);
  auto key = std::make_pair(kernel, dev);
  auto it = cache.find(key);
  if (it != cache.end()) return it->second;
  int per_cu = 0, cus = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, block, dyn_lds) !=
          hipSuccess ||
      per_cu < 1)
    per_cu = 1;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus < 1)
    cus = 256;
  const int64_t r = (int64_t)per_cu * cus;
  cache[key] = r;
  return r;
}

}  // namespace pqm

namespace {

bool aligned(const void *p, size_t a) { return ((uintptr_t)p % a) == 0; }

pqm_status from_hip(hipError_t e) { return e == hipSuccess ? PQM_OK : PQM_ERR_HIP; }

}  // namespace

extern "C" {

const char *pqm_status_string(pqm_status s) {
  switch (s) {
    case PQM_OK: return "ok";
    case PQM_ERR_NULL: return "required pointer is NULL";
    case PQM_ERR_SHAPE: return "invalid shape or size";
    case PQM_ERR_ALIGN: return "pointer or stride not 16-byte aligned";
    case PQM_ERR_ENUM: return "unknown or unsupported format/kind/dtype";
    case PQM_ERR_WORKSPACE: return "workspace too small";
    case PQM_ERR_HIP: return "HIP launch failed";
  }
  return "unknown status";
}

int pqm_abi_version(void) { return 1; }

pqm_status pqm_quantize_mxfp8(const uint16_t *x, int64_t rows, int64_t cols, int64_t ld,
                              uint8_t *q_row, uint8_t *s_row, uint8_t *q_colT,
                              uint8_t *s_colT, hipStream_t stream) {
  const bool row = q_row || s_row, col = q_colT || s_colT;
  if (rows < 0 || cols < 0 || ld < cols || cols % 32) return PQM_ERR_SHAPE;
  if (rows == 0 || cols == 0) return PQM_OK;
  if (!x) return PQM_ERR_NULL;
  if (!row && !col) return PQM_ERR_NULL;
  if (row && (!q_row || !s_row)) return PQM_ERR_NULL;
  if (col && (!q_colT || !s_colT)) return PQM_ERR_NULL;
  if (col && rows % 32) return PQM_ERR_SHAPE;
  if (((rows + 127) / 128) * ((cols + 127) / 128) >= ((int64_t)1 << 31)) return PQM_ERR_SHAPE;
  if (!aligned(x, 16) || ld % 8) return PQM_ERR_ALIGN;
  if (row && (!aligned(q_row, 16) || !aligned(s_row, 4))) return PQM_ERR_ALIGN;
  if (col && (!aligned(q_colT, 16) || !aligned(s_colT, 4))) return PQM_ERR_ALIGN;
  return from_hip(pqm::launch_quantize_mxfp8(x, rows, cols, ld, row ? q_row : nullptr, s_row,
                                             col ? q_colT : nullptr, s_colT, stream));
}

pqm_status pqm_quantize_fp8_block(const uint16_t *x, int64_t rows, int64_t cols, int64_t ld,
                                  int64_t block_rows, uint8_t *q, float *s,
                                  hipStream_t stream) {
  if (block_rows != 1 && block_rows != 128) return PQM_ERR_SHAPE;
  if (rows < 0 || cols < 0 || ld < cols || cols % 128 || rows % block_rows) return PQM_ERR_SHAPE;
  if (rows == 0 || cols == 0) return PQM_OK;
  const int64_t units = block_rows == 1 ? (rows * ((cols + 511) / 512) + 3) / 4
                                        : (rows / 128) * (cols / 128);
  if (units >= ((int64_t)1 << 31)) return PQM_ERR_SHAPE;
  if (!x || !q || !s) return PQM_ERR_NULL;
  if (!aligned(x, 16) || ld % 8 || !aligned(q, 8) || !aligned(s, 4)) return PQM_ERR_ALIGN;
  return from_hip(pqm::launch_quantize_fp8_block(x, rows, cols, ld, block_rows, q, s, stream));
}

size_t pqm_quantize_nvfp4_workspace(int64_t rows, int64_t cols, int64_t rows_per_scale) {
  (void)cols;
  if (rows <= 0 || rows_per_scale <= 0) return 0;
  return pqm::nvfp4_workspace_bytes(rows, rows_per_scale);
}

pqm_status pqm_quantize_nvfp4_per_token(const uint16_t *x, int64_t rows, int64_t cols,
                                        int64_t ld, int64_t rows_per_scale, uint8_t *q,
                                        uint8_t *s_block, float *s_outer, void *workspace,
                                        size_t workspace_bytes, hipStream_t stream) {
  if (rows < 0 || cols < 0 || ld < cols || cols % 16 || rows_per_scale < 1)
    return PQM_ERR_SHAPE;
  if (rows % rows_per_scale) return PQM_ERR_SHAPE;
  if (cols > pqm::nvfp4_max_cols() || rows >= ((int64_t)1 << 31)) return PQM_ERR_SHAPE;
  if (rows > 0 && (!x || !q || !s_block || !s_outer)) return PQM_ERR_NULL;
  if (rows > 0 && (!aligned(x, 16) || ld % 8 || !aligned(q, 8))) return PQM_ERR_ALIGN;
  if (rows > 0 && !aligned(s_outer, 4)) return PQM_ERR_ALIGN;
  const size_t need = pqm::nvfp4_workspace_bytes(rows, rows_per_scale);
  if (need) {
    if (!workspace) return PQM_ERR_NULL;
    if (workspace_bytes < need) return PQM_ERR_WORKSPACE;
    if (!aligned(workspace, 4)) return PQM_ERR_ALIGN;
  }
  return from_hip(pqm::launch_quantize_nvfp4(x, rows, cols, ld, rows_per_scale, q, s_block,
                                             s_outer, workspace, stream));
}

pqm_status pqm_dequantize(pqm_format fmt, const uint8_t *q, const uint8_t *s_block,
                          const float *s_outer, int64_t rows, int64_t cols,
                          int64_t rows_per_scale, uint16_t *y, hipStream_t stream) {
  if (fmt != PQM_FMT_MXFP8 && fmt != PQM_FMT_NVFP4) return PQM_ERR_ENUM;
  if (rows < 0 || cols < 0) return PQM_ERR_SHAPE;
  if (fmt == PQM_FMT_MXFP8 && cols % 32) return PQM_ERR_SHAPE;
  if (fmt == PQM_FMT_NVFP4) {
    if (cols % 16 || rows_per_scale < 1 || rows % rows_per_scale) return PQM_ERR_SHAPE;
  }
  if (rows == 0 || cols == 0) return PQM_OK;
  if (!q || !s_block || !y) return PQM_ERR_NULL;
  if (fmt == PQM_FMT_NVFP4 && !s_outer) return PQM_ERR_NULL;
  if (!aligned(y, 16)) return PQM_ERR_ALIGN;
  if (fmt == PQM_FMT_MXFP8 && !aligned(q, 16)) return PQM_ERR_ALIGN;
  if (fmt == PQM_FMT_NVFP4 && (!aligned(q, 8) || !aligned(s_outer, 4))) return PQM_ERR_ALIGN;
  return from_hip(pqm::launch_dequantize((int)fmt, q, s_block, s_outer, rows, cols,
                                         rows_per_scale, y, stream));
}

pqm_status pqm_moe_grouped_gemm(pqm_format fmt, pqm_gemm_kind kind, const void *a,
                                const uint8_t *a_scale, const float *a_outer, const void *b,
                                const uint8_t *b_scale, const float *b_outer,
                                int64_t b_rows_per_scale, const float *bias,
                                const int64_t *offsets, int64_t G,
                                int64_t M_total, int64_t N, int64_t K, void *out,
                                pqm_dtype out_dtype, void *workspace, size_t workspace_bytes,
                                hipStream_t stream) {
  if (fmt != PQM_FMT_BF16 && fmt != PQM_FMT_MXFP8 && fmt != PQM_FMT_NVFP4 &&
      fmt != PQM_FMT_FP8_BLOCK)
    return PQM_ERR_ENUM;
  if (kind != PQM_GEMM_FPROP && kind != PQM_GEMM_DGRAD && kind != PQM_GEMM_WGRAD)
    return PQM_ERR_ENUM;
  if (out_dtype != PQM_OUT_BF16 && out_dtype != PQM_OUT_FP32) return PQM_ERR_ENUM;
  if ((fmt == PQM_FMT_NVFP4 || fmt == PQM_FMT_FP8_BLOCK) && kind != PQM_GEMM_FPROP)
    return PQM_ERR_ENUM;
  if (bias && kind != PQM_GEMM_FPROP) return PQM_ERR_ENUM;  // the forward epilogue's term
  if (G < 0 || M_total < 0 || N < 0 || K < 0) return PQM_ERR_SHAPE;
  if (fmt == PQM_FMT_MXFP8 && kind != PQM_GEMM_WGRAD && K % 32) return PQM_ERR_SHAPE;
  if (fmt == PQM_FMT_MXFP8 && kind == PQM_GEMM_DGRAD &&
      (K % 128 || K > 2048 || G * K * 256 + K >= ((int64_t)1 << 32)))
    return PQM_ERR_SHAPE;
  if (fmt == PQM_FMT_MXFP8 && kind == PQM_GEMM_WGRAD &&
      (M_total % 32 || M_total * 256 + 4096 >= ((int64_t)1 << 32)))
    return PQM_ERR_SHAPE;
  if (fmt == PQM_FMT_NVFP4 && K % 16) return PQM_ERR_SHAPE;
  if (fmt == PQM_FMT_FP8_BLOCK && (K % 128 || K > 8192 || N % 128)) return PQM_ERR_SHAPE;
  if (fmt == PQM_FMT_BF16 && (K % 8 || N % 8)) return PQM_ERR_SHAPE;
  if (fmt == PQM_FMT_NVFP4 && (b_rows_per_scale < 1 || (G * N) % b_rows_per_scale))
    return PQM_ERR_SHAPE;
  if (G == 0) return PQM_OK;
  // operands are read only when the contraction is non-empty; the output is
  // written only when it has elements (K = 0 clears the routed rows)
  const bool reads = M_total > 0 && N > 0 && K > 0;
  const bool writes = kind == PQM_GEMM_WGRAD ? (N > 0 && K > 0) : (M_total > 0 && N > 0);
  if (!offsets || (writes && !out)) return PQM_ERR_NULL;
  if (reads && (!a || !b)) return PQM_ERR_NULL;
  if (reads && (fmt == PQM_FMT_MXFP8 || fmt == PQM_FMT_NVFP4) && (!a_scale || !b_scale))
    return PQM_ERR_NULL;
  if (reads && (fmt == PQM_FMT_NVFP4 || fmt == PQM_FMT_FP8_BLOCK) && (!a_outer || !b_outer))
    return PQM_ERR_NULL;
  if (!aligned(a, 16) || !aligned(b, 16) || !aligned(out, 16) || !aligned(offsets, 8) ||
      !aligned(bias, 4))
    return PQM_ERR_ALIGN;
  if (fmt == PQM_FMT_MXFP8 && (!aligned(a_scale, 4) || !aligned(b_scale, 4)))
    return PQM_ERR_ALIGN;
  if (fmt == PQM_FMT_FP8_BLOCK && (!aligned(a_outer, 4) || !aligned(b_outer, 4)))
    return PQM_ERR_ALIGN;
  // the workspace is optional; one that is too small or misaligned is unused
  const int64_t ws_need = pqm::grouped_gemm_workspace_bytes((int)fmt, (int)kind);
  uint32_t *ctr = ws_need > 0 && workspace && (int64_t)workspace_bytes >= ws_need &&
                          aligned(workspace, 4)
                      ? static_cast<uint32_t *>(workspace)
                      : nullptr;
  return from_hip(pqm::launch_grouped_gemm((int)fmt, (int)kind, a, a_scale, a_outer, b, b_scale,
                                           b_outer, b_rows_per_scale, offsets, G, M_total, N,
                                           K, out, out_dtype == PQM_OUT_FP32, bias, ctr, stream));
}

size_t pqm_moe_grouped_gemm_workspace_size(pqm_format fmt, pqm_gemm_kind kind) {
  return (size_t)pqm::grouped_gemm_workspace_bytes((int)fmt, (int)kind);
}

pqm_status pqm_moe_fc2_online_nvfp4(const uint16_t *p, const uint8_t *w_q,
                                    const uint8_t *w_scale, const float *w_outer,
                                    int64_t w_rows_per_scale, const int64_t *offsets,
                                    int64_t G, int64_t M_total, int64_t N, int64_t K,
                                    void *out, pqm_dtype out_dtype, float *gs_out,
                                    uint8_t *q_out, uint8_t *sb_out, hipStream_t stream) {
  if (out_dtype != PQM_OUT_BF16 && out_dtype != PQM_OUT_FP32) return PQM_ERR_ENUM;
  if (G < 0 || M_total < 0 || N < 0 || K <= 0 || K % 256) return PQM_ERR_SHAPE;
  if (w_rows_per_scale < 1 || (G * N) % w_rows_per_scale) return PQM_ERR_SHAPE;
  if (G == 0 || M_total == 0 || N == 0) return PQM_OK;
  if (!p || !w_q || !w_scale || !w_outer || !offsets || !out) return PQM_ERR_NULL;
  if ((q_out == nullptr) != (sb_out == nullptr)) return PQM_ERR_NULL;
  if (!aligned(p, 16) || !aligned(w_q, 16) || !aligned(out, 16) || !aligned(q_out, 16) ||
      !aligned(offsets, 8) || !aligned(w_scale, 4) || !aligned(gs_out, 4))
    return PQM_ERR_ALIGN;
  return from_hip(pqm::launch_fc2_online_nvfp4(p, w_q, w_scale, w_outer, w_rows_per_scale,
                                               offsets, G, M_total, N, K, out,
                                               out_dtype == PQM_OUT_FP32, gs_out, q_out, sb_out,
                                               stream));
}

pqm_status pqm_moe_fc2_online_nvfp4_split(const uint16_t *p, const uint8_t *w_q,
                                          const uint8_t *w_scale, const float *w_outer,
                                          int64_t w_rows_per_scale, const int64_t *offsets,
                                          int64_t G, int64_t M_total, int64_t N, int64_t K,
                                          void *out, pqm_dtype out_dtype, float *gs_out,
                                          uint8_t *q_out, uint8_t *sb_out, float *ratio_out,
                                          hipStream_t stream) {
  if (out_dtype != PQM_OUT_BF16 && out_dtype != PQM_OUT_FP32) return PQM_ERR_ENUM;
  if (G < 0 || M_total < 0 || N < 0 || K <= 0 || K % 256 || K > 4096) return PQM_ERR_SHAPE;
  if (w_rows_per_scale < 1 || (G * N) % w_rows_per_scale) return PQM_ERR_SHAPE;
  if (G == 0 || M_total == 0 || N == 0) return PQM_OK;
  if (!p || !w_q || !w_scale || !w_outer || !offsets || !out || !gs_out || !q_out || !sb_out ||
      !ratio_out)
    return PQM_ERR_NULL;
  if (!aligned(p, 16) || !aligned(w_q, 16) || !aligned(out, 16) || !aligned(q_out, 16) ||
      !aligned(offsets, 8) || !aligned(w_scale, 4) || !aligned(sb_out, 4) ||
      !aligned(gs_out, 4) || !aligned(ratio_out, 4))
    return PQM_ERR_ALIGN;
  return from_hip(pqm::launch_fc2_online_nvfp4_split(p, w_q, w_scale, w_outer, w_rows_per_scale,
                                                     offsets, G, M_total, N, K, out,
                                                     out_dtype == PQM_OUT_FP32, gs_out, q_out,
                                                     sb_out, ratio_out, stream));
}

pqm_status pqm_moe_gemm_swiglu_quantize_mxfp8(const uint8_t *a, const uint8_t *a_scale,
                                              const uint8_t *b, const uint8_t *b_scale,
                                              const int64_t *offsets, int64_t G, int64_t M_total,
                                              int64_t inter, int64_t K, const float *prob,
                                              const int32_t *src, uint8_t *q, uint8_t *s,
                                              hipStream_t stream) {
  if (G < 0 || M_total < 0 || inter < 0 || K < 0) return PQM_ERR_SHAPE;
  if (inter % 128 || K % 128 || K / 32 > 64) return PQM_ERR_SHAPE;
  if (G == 0 || M_total == 0 || inter == 0) return PQM_OK;
  if (K == 0) return PQM_ERR_SHAPE;
  if (!a || !a_scale || !b || !b_scale || !offsets || !prob || !q || !s) return PQM_ERR_NULL;
  if (!aligned(a, 16) || !aligned(b, 16) || !aligned(q, 16) || !aligned(offsets, 8) ||
      !aligned(a_scale, 4) || !aligned(b_scale, 4))
    return PQM_ERR_ALIGN;
  return from_hip(pqm::launch_gemm_swiglu_mxfp8(a, a_scale, b, b_scale, offsets, G, M_total,
                                                inter, K, prob, src, q, s, stream));
}

}  // extern "C"
