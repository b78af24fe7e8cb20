/*
 * pqmoe.h -- C ABI of the block-scaled quantizer and MoE grouped-GEMM
 * library for AMD Instinct MI355X (gfx950).
 *
 * The library implements the data-parallel core of the low-precision RL
 * precision contract described in:
 *   [BW] "Towards Blackwell-Native 8-bit and 4-bit RL"
 *   [MT] "miniTE technical report: stable training and efficient
 *        implementation of native NVFP4 RL"
 *   [PR] "PR #2396 report: docs: refresh MXFP8 and NVFP4 RL guide"
 *
 * Conventions for every entry point
 * ---------------------------------
 *  - Pointers named d_* or documented as "device" are device pointers (HBM);
 *    the caller owns every buffer.  The library never allocates, frees or
 *    synchronizes; all work is enqueued on `stream` (NULL = the null stream)
 *    and returns before it runs.
 *  - bf16 tensors are passed as 16-bit bit patterns (uint16_t).  Inputs must
 *    be finite; NaN and infinity are outside the contract.
 *  - Shapes are row-major.  `ld` is the row stride of an input in elements.
 *  - Argument errors are reported synchronously, before anything is
 *    enqueued: PQM_ERR_NULL (a required pointer is NULL), PQM_ERR_SHAPE
 *    (a size is negative or not a multiple of the block length),
 *    PQM_ERR_ALIGN (a vector-loaded pointer or stride is not 16-byte
 *    aligned), PQM_ERR_ENUM (unknown format/kind/dtype), PQM_ERR_WORKSPACE
 *    (workspace too small).  A failed launch returns PQM_ERR_HIP.
 *  - Results are deterministic: the same inputs give bitwise identical
 *    outputs on every run (fixed reduction order, no split-K atomics),
 *    following the deterministic-mode rule of [MT] 4.5.
 *  - Zero-sized inputs (rows == 0, or an empty group) are legal and enqueue
 *    nothing for the empty part.
 */
#ifndef PQMOE_H
#define PQMOE_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum pqm_status {
    PQM_OK = 0,
    PQM_ERR_NULL = 1,
    PQM_ERR_SHAPE = 2,
    PQM_ERR_ALIGN = 3,
    PQM_ERR_ENUM = 4,
    PQM_ERR_WORKSPACE = 5,
    PQM_ERR_HIP = 6
} pqm_status;

typedef enum pqm_format {
    PQM_FMT_BF16 = 0,  /* plain bf16 operands */
    PQM_FMT_MXFP8 = 1, /* E4M3 data, one E8M0 scale per 32 along the row */
    PQM_FMT_NVFP4 = 2, /* packed E2M1, one E4M3 scale per 16, FP32 outer */
    PQM_FMT_FP8_BLOCK = 3 /* E4M3, FP32 scale per 1x128 tile / 128x128 block */
} pqm_format;

typedef enum pqm_gemm_kind {
    PQM_GEMM_FPROP = 0, /* Y[m,:] = A[m,:] . B_g^T,  B [G, N, K]          */
    PQM_GEMM_DGRAD = 1, /* Y[m,:] = A[m,:] . B_g,    B [G, K, N] (bf16)   */
    PQM_GEMM_WGRAD = 2  /* Y_g = A_g^T . B_g over the group's rows (bf16) */
} pqm_gemm_kind;

typedef enum pqm_dtype {
    PQM_OUT_BF16 = 0,
    PQM_OUT_FP32 = 1
} pqm_dtype;

/* Human-readable name of a status code (static string, never NULL). */
const char *pqm_status_string(pqm_status s);

/* Version of the ABI described by this header. */
int pqm_abi_version(void);

/*
 * MXFP8 quantization ([BW] Format background: MXFP8; Recipe 1: training).
 *
 * Each 1x32 block of E4M3 values shares one E8M0 (power of two) scale,
 * rounded up so the block maximum is never clipped: the scale is 2^e with
 * e the smallest integer for which max|x| <= 448 * 2^e (e >= -127; an
 * all-zero block gets e = -127).  Elements are x / 2^e rounded to the
 * nearest E4M3 value, ties to even; a negative input that rounds to zero
 * keeps its sign (0x80).
 *
 * Row-wise and column-wise copies are both quantized independently from
 * the bf16 input in the same pass (never one from the other):
 *   x       [rows, cols] bf16, row stride ld elements           (device)
 *   q_row   [rows, cols]       E4M3 bytes, 1x32 blocks along rows  (device)
 *   s_row   [rows, cols/32]    E8M0 bytes                          (device)
 *   q_colT  [cols, rows]       E4M3 bytes of the 32x1 blocks down each
 *                              column, stored transposed so each block is
 *                              contiguous                          (device)
 *   s_colT  [cols, rows/32]    E8M0 bytes                          (device)
 * Either output pair may be NULL to skip that copy, not both.
 * Requires cols % 32 == 0; rows % 32 == 0 when the column copy is asked
 * for; fewer than 2^31 tiles of 128 x 128 (PQM_ERR_SHAPE otherwise); x,
 * q_row, q_colT and ld 16-byte aligned (ld % 8 == 0); s_row and s_colT
 * 4-byte aligned (PQM_ERR_ALIGN otherwise).
 */
pqm_status pqm_quantize_mxfp8(const uint16_t *x, int64_t rows, int64_t cols,
                              int64_t ld, uint8_t *q_row, uint8_t *s_row,
                              uint8_t *q_colT, uint8_t *s_colT,
                              hipStream_t stream);

/*
 * NVFP4 quantization with an online FP32 outer scale ([BW] Format
 * background: NVFP4; Recipe 2: per-token activation scaling, gate/up
 * pairing; [MT] 2.2 decode x^ = q s_b s_g; [MT] 5.6 gs = gamax / 2688).
 *
 * Rows are split into scope groups of `rows_per_scale` consecutive rows;
 * each group has one FP32 outer scale s_g:
 *   rows_per_scale = 1    per token (the activation recipe): one fused pass
 *                         reads each row once and writes all three outputs;
 *   rows_per_scale = R_e  one scale per expert tensor; for fused gate/up
 *                         weights [gate; up] of R_e rows this is the joint
 *                         option: gate and up share one outer scale.
 * For a group with absolute maximum A:
 *   s_g   = A / 2688 rounded once to binary32 (2688 = 6 * 448);
 *   s_b   = nearest E4M3 to a_b / (6 s_g) for each 1x16 block with block
 *           maximum a_b, ties to even, saturating at 448 (0 if s_g == 0);
 *   q     = nearest E2M1 to x / (s_b s_g), ties to even, saturating at 6
 *           (+-0 if s_b == 0); all quotients are exact, not approximated.
 * Outputs (device):
 *   q        [rows, cols/2]  packed E2M1, element 2j in the low nibble
 *   s_block  [rows, cols/16] E4M3 bytes
 *   s_outer  [rows / rows_per_scale] binary32 decode scales s_g
 * Requires cols % 16 == 0, cols <= 16384, rows < 2^31, rows % rows_per_scale
 * == 0, x and ld 16-byte aligned, q 8-byte aligned, s_outer 4-byte aligned
 * (PQM_ERR_SHAPE / PQM_ERR_ALIGN otherwise).  When rows_per_scale > 1 the group maximum is reduced across
 * workgroups through `workspace` (device, >= pqm_quantize_nvfp4_workspace
 * bytes, 4-byte aligned; contents on entry are ignored); it may be NULL
 * when rows_per_scale == 1.
 */
pqm_status pqm_quantize_nvfp4_per_token(const uint16_t *x, int64_t rows,
                                        int64_t cols, int64_t ld,
                                        int64_t rows_per_scale, uint8_t *q,
                                        uint8_t *s_block, float *s_outer,
                                        void *workspace,
                                        size_t workspace_bytes,
                                        hipStream_t stream);

/* Workspace bytes pqm_quantize_nvfp4_per_token needs for these sizes. */
size_t pqm_quantize_nvfp4_workspace(int64_t rows, int64_t cols,
                                    int64_t rows_per_scale);

/*
 * Block-scaled FP8 in the DeepSeek-V3 style ([BW] Why Blackwell-native
 * recipes: 128x128 weight blocks and 1x128 activation tiles, an FP32 scale
 * per block computed online and applied around the matrix core; [PR] Choose
 * a precision: FP8 block-wise, 128x128, FP32 scales).
 *
 * Blocks of block_rows x 128 (block_rows = 1: activation tiles; 128: weight
 * blocks).  For a block with absolute maximum A:
 *   s = A / 448 rounded once to binary32;
 *   q = nearest E4M3 to the exact quotient x / s, ties to even, saturating
 *       at 448 (the block maximum encodes to +-448); A = 0 gives s = 0 and
 *       q = +-0 (a negative input keeps its sign: 0x80).
 *   x [rows, cols] bf16, row stride ld elements                  (device)
 *   q [rows, cols] E4M3 bytes                                    (device)
 *   s [rows / block_rows, cols / 128] binary32                   (device)
 * Requires block_rows 1 or 128, cols % 128 == 0, rows % block_rows == 0,
 * fewer than 2^31 workgroups (PQM_ERR_SHAPE); x and ld 16-byte aligned,
 * q 8-byte and s 4-byte aligned (PQM_ERR_ALIGN).
 */
pqm_status pqm_quantize_fp8_block(const uint16_t *x, int64_t rows, int64_t cols, int64_t ld,
                                  int64_t block_rows, uint8_t *q, float *s,
                                  hipStream_t stream);

/*
 * Dequantize to bf16 for the dequantized-backward mode ([BW]
 * High-precision and dequantized backward: the backward GEMMs run in BF16
 * on the BF16 dequantization of the exact forward operands).
 *
 * y = the exact decoded value rounded once to the nearest bf16 (ties to
 * even; values beyond bf16 range become +-inf):
 *   PQM_FMT_MXFP8: q [rows, cols] E4M3, s_block [rows, cols/32] E8M0,
 *                  s_outer unused (may be NULL);  y = q * 2^(s - 127)
 *   PQM_FMT_NVFP4: q [rows, cols/2] packed E2M1, s_block [rows, cols/16]
 *                  E4M3, s_outer [rows / rows_per_scale] binary32;
 *                  y = q * s_b * s_g
 * y [rows, cols] bf16 (device).  The orientation of y is that of q: a
 * column-wise (transposed) MXFP8 copy dequantizes to the transpose.
 * Requires cols % 32 == 0 (MXFP8) or cols % 16 == 0 (NVFP4).
 */
pqm_status pqm_dequantize(pqm_format fmt, const uint8_t *q,
                          const uint8_t *s_block, const float *s_outer,
                          int64_t rows, int64_t cols, int64_t rows_per_scale,
                          uint16_t *y, hipStream_t stream);

/*
 * Grouped GEMM over routed experts ([MT] 5.2: one contiguous buffer with
 * expert offsets handed to a dense grouped GEMM, metadata on the device,
 * empty experts handled inside; [MT] 5.4: ACC = block-scaled GEMM(A, B),
 * ACC *= alpha_a[m] (* alpha_b)).
 *
 * offsets [G+1] int64 (device): group g owns rows offsets[g] ..
 * offsets[g+1]-1 of A; offsets[0] = 0, non-decreasing, offsets[G] <=
 * M_total (rows from offsets[G] on are neither read nor written).  Empty
 * groups are legal.  Values outside this contract are undefined behaviour.
 *
 *   PQM_GEMM_FPROP (all formats):   Y[m, n] = sum_k A[m, k] B_g[n, k]
 *       A [M_total, K] and B [G, N, K], both with K contiguous;
 *       Y [M_total, N].
 *   PQM_GEMM_DGRAD (PQM_FMT_BF16):  Y[m, n] = sum_k A[m, k] B_g[k, n]
 *       A [M_total, K], B [G, K, N] (N contiguous); Y [M_total, N].
 *   PQM_GEMM_WGRAD (PQM_FMT_BF16):  Y_g[n, k] = sum_{m in g} A[m, n] B[m, k]
 *       A [M_total, N], B [M_total, K]; Y [G, N, K] (zero for empty g).
 *   PQM_GEMM_DGRAD (PQM_FMT_MXFP8): the same Y, with the contraction
 *       blocks of B_g running along k ([BW] MXFP8 training: backward GEMMs
 *       read the column-wise copies): a = row-wise MXFP8 of A [M_total, K];
 *       b / b_scale = the column-wise copy (q_colT [N, G*K], s_colT
 *       [N, G*K/32]) that pqm_quantize_mxfp8 makes of the stacked B [G*K, N];
 *       expert g uses its columns g*K .. g*K+K-1.  K % 128 == 0, K <= 2048,
 *       G*K*256 + K < 2^32.
 *   PQM_GEMM_WGRAD (PQM_FMT_MXFP8): the same Y_g from the column-wise
 *       copies of both operands: a / a_scale = q_colT [N, M_total] /
 *       s_colT [N, M_total/32] of A, b / b_scale = q_colT [K, M_total] /
 *       s_colT [K, M_total/32] of B.  Every offsets[g] must be a multiple
 *       of 32 (each expert's rows padded to whole 32-row blocks, padding
 *       rows zero), else the result is undefined (reads stay in bounds).
 *       M_total % 32 == 0, M_total*256 + 4096 < 2^32; any N, K.
 *
 * Operand encodings (all device):
 *   PQM_FMT_BF16:  a, b bf16; scales and outer scales unused (NULL).
 *   PQM_FMT_MXFP8: a = E4M3 [M_total, K], a_scale = E8M0 [M_total, K/32];
 *                  b = E4M3 [G, N, K], b_scale = E8M0 [G, N, K/32].
 *   PQM_FMT_NVFP4: a = packed E2M1 [M_total, K/2], a_scale = E4M3
 *                  [M_total, K/16], a_outer = binary32 [M_total] (per
 *                  token); b = packed E2M1 [G, N, K/2], b_scale = E4M3
 *                  [G, N, K/16], b_outer = binary32 [(G*N) /
 *                  b_rows_per_scale] (b_rows_per_scale = N: one scale per
 *                  expert, e.g. joint gate/up).
 *   PQM_FMT_FP8_BLOCK (FPROP only; [BW] Why Blackwell-native recipes: the
 *                  DeepSeek-V3 design, FP32 scales applied around the
 *                  matrix core): a = E4M3 [M_total, K] with a_outer =
 *                  binary32 [M_total, K/128] (1x128 tiles); b = E4M3
 *                  [G, N, K] with b_outer = binary32 [G*N/128, K/128]
 *                  (128x128 blocks), as pqm_quantize_fp8_block makes them;
 *                  a_scale, b_scale unused.  Y[m, n] = sum over 128-K
 *                  blocks kb of a_outer[m, kb] b_outer[n/128, kb] times the
 *                  block's sum of E4M3 products.  K % 128 == 0, K <= 8192,
 *                  N % 128 == 0.
 * a, b and out 16-byte aligned, offsets 8-byte aligned, MXFP8 scale arrays
 * and block-FP8 scales 4-byte aligned (PQM_ERR_ALIGN otherwise).
 * The products use the exact operand values; accumulation is binary32 and
 * the outer scales are applied to the binary32 accumulator.
 * out: Y in bf16 (rounded once) or binary32 per out_dtype.
 * K % 32 == 0 (MXFP8 FPROP / DGRAD), K % 16 == 0 (NVFP4), K % 8 and
 * N % 8 == 0 (BF16); BF16 WGRAD needs N % 8 == 0 and K % 8 == 0; NVFP4 and
 * block FP8 are FPROP only (PQM_ERR_ENUM otherwise).
 * workspace (device, optional): pqm_moe_grouped_gemm_workspace_size(fmt,
 * kind) bytes, 4-byte aligned, contents irrelevant; the call overwrites
 * them, so calls that may run at the same time need separate workspaces.
 * Only the MXFP8 weight gradient uses one today (a tile counter: with it the
 * tiles, heaviest experts first, go to whichever workgroup is free; without
 * it they are dealt in a fixed order, same results either way).  NULL / 0,
 * or a buffer that is too small or misaligned, means no workspace.
 * bias (device, optional; FPROP only, else PQM_ERR_ENUM; 4-byte aligned):
 * binary32 [G, N], the forward epilogue's additive term ([MT] 5.4: the
 * accumulator times the outer scales, plus bias): Y_g[m, n] = alpha
 * x accumulator + bias[g, n] in binary32 (NVFP4: the product and the sum
 * in binary64, rounded once to binary32), then the output rounding.  NULL:
 * no bias.
 * An empty contraction (K == 0) makes FPROP / DGRAD write zeros (with a
 * bias: each routed row's bias row) to rows 0 .. offsets[G]-1 and read no
 * operand; operand, scale and outer-scale pointers are required (non-NULL)
 * only when M_total, N and K are all positive, and out only when Y has
 * elements.
 */
pqm_status pqm_moe_grouped_gemm(pqm_format fmt, pqm_gemm_kind kind,
                                const void *a, const uint8_t *a_scale,
                                const float *a_outer, const void *b,
                                const uint8_t *b_scale, const float *b_outer,
                                int64_t b_rows_per_scale, const float *bias,
                                const int64_t *offsets, int64_t G,
                                int64_t M_total, int64_t N, int64_t K,
                                void *out, pqm_dtype out_dtype,
                                void *workspace, size_t workspace_bytes,
                                hipStream_t stream);

/* Workspace bytes pqm_moe_grouped_gemm can use for (fmt, kind): 4 for the
 * MXFP8 weight gradient, 0 otherwise (host only, no device work). */
size_t pqm_moe_grouped_gemm_workspace_size(pqm_format fmt, pqm_gemm_kind kind);

/*
 * The NVFP4 down projection with online amax compensation ([MT] 5.6, the
 * single-pass fusion study): the activation P is consumed in 128-wide K-tiles
 * before each row's full maximum is known.  Per row, a running maximum
 * gamax = max(|P| over the tiles so far); tile i is encoded under
 * gs = binary32(gamax / 2688) exactly as pqm_quantize_nvfp4_per_token
 * encodes a row of maximum gamax (1x16 E4M3 block scales, E2M1 codes), its
 * block-scaled product with W2 (without gs) is dO_i, and the accumulator
 * moves to the new scale: O = O (gs_prev / gs) + dO_i, gs_prev = gs.  While
 * gamax is zero the tile adds nothing and gs_prev stays.  Y = O gs_prev
 * alpha_W2(n); an all-zero row gives zero.  The encodings depend on when the
 * row's maximum arrives, so Y can differ from the two-pass path (whole-row
 * per-token encoding, then pqm_moe_grouped_gemm NVFP4) by the quantization
 * difference, while the compensation itself is exact up to rounding.
 *   p        bf16 [M_total, K], routed rows grouped by offsets;
 *   w_q      packed E2M1 [G, N, K/2], w_scale E4M3 [G, N, K/16] (4-byte
 *            aligned), w_outer binary32 [(G*N) / w_rows_per_scale];
 *   out      [M_total, N] bf16 (rounded once) or binary32 per out_dtype;
 *            rows 0 .. offsets[G]-1 written;
 *   gs_out   (optional, binary32 [M_total]) each row's final gs;
 *   q_out, sb_out (optional, both or neither; [M_total, K/2] and
 *            [M_total, K/16]) the codes and block scales P was encoded
 *            with, tile by tile.
 * Accumulation is binary32; gs_prev / gs is one binary32 division.
 * K must be a positive multiple of 256 and w_rows_per_scale >= 1 dividing
 * G*N (PQM_ERR_SHAPE); p, w_q, out, q_out 16-byte aligned, offsets 8-byte,
 * w_scale and gs_out 4-byte (PQM_ERR_ALIGN).  The caller owns every buffer;
 * nothing is allocated.
 */
pqm_status pqm_moe_fc2_online_nvfp4(const uint16_t *p, const uint8_t *w_q,
                                    const uint8_t *w_scale, const float *w_outer,
                                    int64_t w_rows_per_scale, const int64_t *offsets,
                                    int64_t G, int64_t M_total, int64_t N, int64_t K,
                                    void *out, pqm_dtype out_dtype, float *gs_out,
                                    uint8_t *q_out, uint8_t *sb_out, hipStream_t stream);

/*
 * The same online-amax FC2 ([MT] 5.6) split into two kernels.  A row's encoding
 * depends on its K-tiles only, not on the output column, so the first kernel
 * encodes every routed row once.  The second is the NVFP4 grouped GEMM
 * on those codes, which moves its accumulator rows by the stored ratios
 * before each K-tile.  The codes, block scales and gs are those of
 * pqm_moe_fc2_online_nvfp4, and so is Y bit for bit: the same accumulation
 * order and the same epilogue.  The one-kernel entry point encodes P again
 * in every 256-column tile.
 *   p, w_q, w_scale, w_outer, offsets, out, out_dtype: as
 *            pqm_moe_fc2_online_nvfp4;
 *   gs_out   binary32 [M_total], each row's final gs (written);
 *   q_out, sb_out [M_total, K/2] and [M_total, K/16], the codes and block
 *            scales P was encoded with (written, then read by the GEMM);
 *   ratio_out binary32 [M_total, K/128], each tile's gs_prev / gs (1 when
 *            the row's maximum did not grow; written, then read).
 * Rows 0 .. offsets[G]-1 of every output are written.  All four buffers
 * are required (PQM_ERR_NULL).  K is a positive multiple of 256 and at most
 * 4096 (PQM_ERR_SHAPE).  p, w_q, out and q_out must be 16-byte aligned,
 * offsets 8-byte, and w_scale, sb_out, gs_out and ratio_out 4-byte
 * (PQM_ERR_ALIGN).  The caller owns every buffer; nothing is allocated.
 */
pqm_status pqm_moe_fc2_online_nvfp4_split(const uint16_t *p, const uint8_t *w_q,
                                          const uint8_t *w_scale, const float *w_outer,
                                          int64_t w_rows_per_scale, const int64_t *offsets,
                                          int64_t G, int64_t M_total, int64_t N, int64_t K,
                                          void *out, pqm_dtype out_dtype, float *gs_out,
                                          uint8_t *q_out, uint8_t *sb_out, float *ratio_out,
                                          hipStream_t stream);

/*
 * The MXFP8 gate_up grouped GEMM with its activation fused into the
 * epilogue ([MT] 5.3-5.4: D = act(gate, up) x prob is produced where C is,
 * and quantized for the down GEMM without another pass; C is not written):
 *   C_g = A . B_g^T as pqm_moe_grouped_gemm FPROP (MXFP8, bf16 output),
 *   D   = pqm_swiglu_prob(C, prob, src),  (q, s) = row-wise MXFP8 of D,
 * with the same bytes as those three calls.  A [M_total, K] E4M3 + a_scale
 * [M_total, K/32]; B [G, 2 inter, K] E4M3 (rows 0..inter-1 gate, then up)
 * + b_scale [G, 2 inter, K/32]; prob / src as pqm_swiglu_prob; q [M_total,
 * inter] E4M3 and s [M_total, inter/32] E8M0 (device).
 * Requires inter % 128 == 0, K % 128 == 0, K <= 2048 (PQM_ERR_SHAPE); a, b,
 * q 16-byte aligned, the scale arrays 4-byte aligned (PQM_ERR_ALIGN).
 */
pqm_status pqm_moe_gemm_swiglu_quantize_mxfp8(const uint8_t *a, const uint8_t *a_scale,
                                              const uint8_t *b, const uint8_t *b_scale,
                                              const int64_t *offsets, int64_t G,
                                              int64_t M_total, int64_t inter, int64_t K,
                                              const float *prob, const int32_t *src,
                                              uint8_t *q, uint8_t *s, hipStream_t stream);

/*
 * MoE glue around the grouped GEMM ([MT] 5.2: quantized rows are placed in
 * one contiguous buffer with offsets marking the expert boundaries, built
 * on the device; [MT] 5.4: D = act(gate, up) x prob; [BW] Fine-grained
 * precision control: routed outputs go through a high-precision weighted
 * reduction).
 */

/*
 * Stable counting sort of token -> expert assignments.
 *   topk_ids  [tokens, k] int32 expert ids in [0, num_experts)   (device)
 *   shared_expert  0, or 1 to append one more group (index num_experts)
 *             holding every token in order, for an always-active shared
 *             expert run through the same grouped GEMM
 *   offsets   [num_experts + 1 + shared_expert] int64: group e owns
 *             positions offsets[e] .. offsets[e+1]-1              (device)
 *   src_row   [tokens * (k + shared_expert)] int32: the assignment index
 *             t*k + j stored at each position (tokens*k + t for the shared
 *             expert's row of token t); within an expert, flat order is
 *             kept                                               (device)
 *   token     [same] int32: the token of each position           (device)
 *   slot      [tokens, k] int32: position of assignment (t, j)   (device)
 *   workspace >= pqm_moe_route_workspace(...) bytes (0 when tokens == 0;
 *             may then be NULL), 8-byte aligned.
 * num_experts <= 4096, tokens * (k + 1) < 2^31.  Ids outside
 * [0, num_experts) are undefined behaviour.
 */
size_t pqm_moe_route_workspace(int64_t tokens, int64_t k, int64_t num_experts);
pqm_status pqm_moe_route(const int32_t *topk_ids, int64_t tokens, int64_t k,
                         int64_t num_experts, int shared_expert, int64_t *offsets,
                         int32_t *src_row, int32_t *token, int32_t *slot,
                         void *workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * pqm_moe_route without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation): the same kernels and the same outputs
 * as pqm_moe_route, with the (chunk, expert) counts and expert totals kept
 * in a scratch array of PQM_ROUTE_NOALLOC_SCRATCH_BYTES that the library
 * holds on each GPU it runs on until the process ends.  The call allocates
 * and frees nothing.  Requires pqm_moe_route_workspace(tokens, k,
 * num_experts) <= PQM_ROUTE_NOALLOC_SCRATCH_BYTES, i.e. about
 * ceil(tokens k / 256) num_experts 4 + num_experts 8 bytes (PQM_ERR_WORKSPACE
 * otherwise; 65536 tokens x top-8 over 256 experts need 2 MiB, 4096 tokens x
 * top-8 over 256 experts 130 KiB); other arguments and errors as
 * pqm_moe_route; PQM_ERR_HIP if the scratch address cannot be obtained.
 * All calls on one GPU share its scratch array: calls that overlap in time
 * on one GPU (different streams, or host threads) race and must be
 * serialized by the caller; calls in stream order are safe.
 */
#define PQM_ROUTE_NOALLOC_SCRATCH_BYTES ((size_t)4 << 20)
pqm_status pqm_moe_route_noalloc(const int32_t *topk_ids, int64_t tokens, int64_t k,
                                 int64_t num_experts, int shared_expert, int64_t *offsets,
                                 int32_t *src_row, int32_t *token, int32_t *slot,
                                 hipStream_t stream);

/*
 * Row gather: out row i = src row (index[i] / divisor), rows of row_bytes
 * bytes (quantized data, scale bytes or FP32 token scales).  With
 * index = token from pqm_moe_route (divisor 1) this places each token's
 * already-quantized row at its expert-sorted positions: per-row blocks run
 * along K, so gathering quantized rows gives the same bytes as quantizing
 * gathered rows.  index entries must be < src_rows * divisor.
 */
pqm_status pqm_moe_gather_rows(const void *src, int64_t src_rows, int64_t row_bytes,
                               const int32_t *index, int64_t n, int64_t divisor,
                               void *out, hipStream_t stream);

/*
 * Per-expert padding to whole blocks of `align` rows ([MT] 5.3: the
 * permuted FC1 activation is padded before it is quantized; [BW] MXFP8
 * training: the column-wise copies have 32 x 1 blocks down each column, so
 * with align = 32 no block holds two experts' tokens):
 *   padded_offsets[0] = 0, padded_offsets[g+1] = padded_offsets[g] +
 *       ceil(n_g / align) * align,  n_g = offsets[g+1] - offsets[g];
 *   out row padded_offsets[g] + j = src row offsets[g] + j for j < n_g;
 *   every other row of out (the padding, and rows from padded_offsets[G]
 *   to out_rows) is zero.
 *   src [src_rows, row_bytes], out [out_rows, row_bytes]        (device)
 *   offsets, padded_offsets [G+1] int64                         (device)
 * Requires align >= 1, row_bytes % 16 == 0, out_rows >= src_rows + G *
 * (align - 1) (room for any offsets; PQM_ERR_SHAPE otherwise); src and out
 * 16-byte aligned, the offset arrays 8-byte aligned (PQM_ERR_ALIGN).
 * offsets must satisfy the pqm_moe_grouped_gemm contract with offsets[G]
 * <= src_rows.
 */
pqm_status pqm_moe_pad_rows(const void *src, int64_t src_rows, int64_t row_bytes,
                            const int64_t *offsets, int64_t G, int64_t align,
                            int64_t *padded_offsets, void *out, int64_t out_rows,
                            hipStream_t stream);

/*
 * Weighted SwiGLU: d[m, j] = bf16( silu(g) * u * p ) with g = c[m, j],
 * u = c[m, inter + j] (c = [gate | up], bf16 [rows, 2*inter]),
 * silu(z) = z / (1 + exp(-z)), p = prob[src[m]] (prob binary32 indexed by
 * assignment, i.e. src_row from pqm_moe_route; with a shared expert prob
 * holds tokens*k + tokens entries, the last tokens of them 1.0; src may be
 * NULL to index prob by m).  Binary32 math with the hardware exponential
 * and reciprocal (about 1 ulp each before the bf16 rounding); for g <= -64
 * the value is formed as (g u p) e^g with power-of-two range scaling, so
 * that neither e^-g nor e^g leaves the binary32 normal range.
 * d bf16 [rows, inter]; inter % 8 == 0.
 */
pqm_status pqm_swiglu_prob(const uint16_t *c, const float *prob, const int32_t *src,
                           int64_t rows, int64_t inter, uint16_t *d, hipStream_t stream);

/*
 * The weighted SwiGLU above fused with the row-wise MXFP8 quantization of
 * its output, the FC2 operand ([MT] 5.3-5.4: the activation of the FC1
 * output, times the router probability, is quantized for the down GEMM
 * without a separate pass over D; [BW] Format background: MXFP8).
 *   q [rows, inter] E4M3 and s [rows, inter / 32] E8M0 equal
 *   pqm_quantize_mxfp8 (row-wise) of the d that pqm_swiglu_prob returns;
 *   d (bf16 [rows, inter]) is also written when non-NULL.
 * Requires inter % 32 == 0 (PQM_ERR_SHAPE), c and d 16-byte aligned, q
 * 8-byte aligned (PQM_ERR_ALIGN); c, prob, q, s non-NULL (PQM_ERR_NULL).
 */
pqm_status pqm_swiglu_prob_quantize_mxfp8(const uint16_t *c, const float *prob,
                                          const int32_t *src, int64_t rows, int64_t inter,
                                          uint16_t *d, uint8_t *q, uint8_t *s,
                                          hipStream_t stream);

/*
 * The weighted SwiGLU above fused with the per-token NVFP4 quantization of
 * its output, the FC2 operand of the NVFP4 recipe ([MT] 5.3-5.4: the
 * activation times the router probability is quantized where it is
 * produced, the per-token amax taken in the same pass, so D is neither
 * written nor read back; [BW] Recipe 2: per-token activation scaling):
 *   q [rows, inter / 2] packed E2M1, s_block [rows, inter / 16] E4M3 and
 *   s_outer [rows] binary32 equal pqm_quantize_nvfp4_per_token (one scale
 *   per row) of the d that pqm_swiglu_prob returns; d (bf16 [rows, inter])
 *   is also written when non-NULL.
 * Requires inter % 16 == 0, inter <= 16384, rows < 2^31 (PQM_ERR_SHAPE);
 * c and d 16-byte aligned, q 8-byte and s_outer 4-byte aligned
 * (PQM_ERR_ALIGN); c, prob, q, s_block, s_outer non-NULL (PQM_ERR_NULL).
 */
pqm_status pqm_swiglu_prob_quantize_nvfp4(const uint16_t *c, const float *prob,
                                          const int32_t *src, int64_t rows, int64_t inter,
                                          uint16_t *d, uint8_t *q, uint8_t *s_block,
                                          float *s_outer, hipStream_t stream);

/*
 * Opt-in check of an offsets array against the grouped-GEMM contract ([MT]
 * 5.2: experts' rows in one contiguous buffer described by offsets on the
 * device); the GEMMs and the glue never check it themselves, since a bad
 * array is undefined behaviour there.  Scans i = 0 .. G and writes, on the
 * stream, to result (device, 2 x int32): result[0] = the first failing check
 * at the smallest failing index (0: the array is valid), result[1] = that
 * index (-1 when valid).  Checks at index i, in this order:
 *   PQM_OFFSETS_FIRST_NOT_ZERO  i == 0 and offsets[0] != 0
 *   PQM_OFFSETS_DECREASING      i < G and offsets[i + 1] < offsets[i]
 *   PQM_OFFSETS_MISALIGNED      offsets[i] % align != 0 (align = 32 for the
 *                               MXFP8 weight gradient's padded groups, else 1)
 *   PQM_OFFSETS_PAST_END        i == G and offsets[G] > M_total
 * G >= 0, M_total >= 0, align >= 1 (PQM_ERR_SHAPE); offsets 8-byte and result
 * 4-byte aligned (PQM_ERR_ALIGN), both non-NULL (PQM_ERR_NULL).  Reads
 * offsets[0 .. G]; one workgroup.
 */
#define PQM_OFFSETS_FIRST_NOT_ZERO 1
#define PQM_OFFSETS_DECREASING 2
#define PQM_OFFSETS_MISALIGNED 3
#define PQM_OFFSETS_PAST_END 4
pqm_status pqm_validate_offsets(const int64_t *offsets, int64_t G, int64_t M_total,
                                int64_t align, int32_t *result, hipStream_t stream);

/*
 * Combine: out[t, n] = bf16( sum_j y_rows[slot[t, j], n] + shared[t, n] ),
 * summed in binary32 in j order (shared may be NULL).  y_rows, shared, out
 * bf16 with N contiguous; N % 8 == 0.
 */
pqm_status pqm_moe_combine(const uint16_t *y_rows, const int32_t *slot,
                           const uint16_t *shared, int64_t tokens, int64_t k, int64_t N,
                           uint16_t *out, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* PQMOE_H */
