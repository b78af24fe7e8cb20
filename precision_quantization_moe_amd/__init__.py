"""MI355X (gfx950) block-scaled quantizers and MoE grouped GEMM.

Thin Python binding over the C ABI in ``include/pqmoe.h`` (``libpqmoe.so``,
built in-tree by ``precision_quantization_moe_amd.build``).  The functions
here only marshal arguments: they allocate outputs with torch on the
tensor's device and call the library on torch's current stream.  Every step
runs in the library's HIP kernels; if the library is missing, importing the
binding raises instead of falling back to anything else.
"""
from __future__ import annotations

from ._binding import (  # noqa: F401
    FMT_BF16, FMT_FP8_BLOCK, FMT_MXFP8, FMT_NVFP4, GEMM_DGRAD, GEMM_FPROP, GEMM_WGRAD,
    OUT_BF16, OUT_FP32, PqmError, dequantize, lib, moe_combine, moe_gather_rows, moe_pad_rows,
    moe_fc2_online_nvfp4, moe_fc2_online_nvfp4_split, moe_gemm_swiglu_quantize_mxfp8, moe_grouped_gemm, moe_route, moe_route_noalloc, pad_rows_bound, quantize_fp8_block,
    quantize_mxfp8,
    quantize_nvfp4_per_token, swiglu_prob, swiglu_prob_quantize_mxfp8, swiglu_prob_quantize_nvfp4,
    validate_offsets, OFFSETS_FIRST_NOT_ZERO, OFFSETS_DECREASING, OFFSETS_MISALIGNED,
    OFFSETS_PAST_END, LIB_PATH,
)
