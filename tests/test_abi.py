"""The C-ABI library loads and exports every entry point include/pqmoe.h
declares; host-side argument validation returns synchronously (these calls
never reach the device).  CPU only."""
from __future__ import annotations

import ctypes
import os
import re

import pytest

import precision_quantization_moe_amd as pqm
from precision_quantization_moe_amd import _binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pqmoe.h")


def _declared():
    txt = open(HEADER).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(pqm_[a-z0-9_]+)\s*\(", txt)))


def test_library_exports_every_declared_symbol():
    L = pqm.lib()
    names = _declared()
    assert len(names) >= 12
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(_binding.SIGNATURES), "binding covers the header"


def test_abi_version_and_status_strings():
    L = pqm.lib()
    assert L.pqm_abi_version() == 1
    for code in range(7):
        assert L.pqm_status_string(code)
    assert L.pqm_status_string(99) == b"unknown status"


# Fake device addresses: 16-byte aligned values never dereferenced, because
# every call below fails validation before any launch.
A16 = ctypes.c_void_p(0x10000)
BAD = ctypes.c_void_p(0x10002)


def test_quantize_mxfp8_validation():
    L = pqm.lib()
    f = L.pqm_quantize_mxfp8
    assert f(A16, 64, 64, 64, None, None, None, None, None) == 1    # no output
    assert f(A16, 64, 64, 64, A16, None, None, None, None) == 1     # half pair
    assert f(A16, 64, 48, 64, A16, A16, None, None, None) == 2      # cols % 32
    assert f(A16, 48, 64, 64, None, None, A16, A16, None) == 2      # rows % 32
    assert f(A16, 64, 64, 32, A16, A16, None, None, None) == 2      # ld < cols
    assert f(A16, -1, 64, 64, A16, A16, None, None, None) == 2
    assert f(BAD, 64, 64, 64, A16, A16, None, None, None) == 3      # x align
    assert f(A16, 64, 64, 68, A16, A16, None, None, None) == 3      # ld % 8
    assert f(A16, 64, 64, 64, BAD, A16, None, None, None) == 3
    assert f(None, 64, 64, 64, A16, A16, None, None, None) == 1


def test_quantize_nvfp4_validation():
    L = pqm.lib()
    f = L.pqm_quantize_nvfp4_per_token
    assert f(A16, 64, 40, 40, 1, A16, A16, A16, None, 0, None) == 2   # cols % 16
    assert f(A16, 64, 64, 64, 3, A16, A16, A16, A16, 4096, None) == 2  # rows % rps
    assert f(A16, 64, 64, 64, 0, A16, A16, A16, None, 0, None) == 2
    assert f(A16, 64, 64, 64, 1, None, A16, A16, None, 0, None) == 1
    assert f(A16, 64, 64, 64, 32, A16, A16, A16, None, 0, None) == 1   # ws needed
    need = L.pqm_quantize_nvfp4_workspace(64, 64, 32)
    assert need == 2 * 16 * 128   # 2 groups x 16 max slots, one 128-byte line each
    assert f(A16, 64, 64, 64, 32, A16, A16, A16, A16, need - 1, None) == 5
    assert f(BAD, 64, 64, 64, 1, A16, A16, A16, None, 0, None) == 3
    assert f(A16, 64, 1 << 20, 1 << 20, 1, A16, A16, A16, None, 0, None) == 2
    assert L.pqm_quantize_nvfp4_workspace(64, 64, 1) == 0


def test_dequantize_validation():
    L = pqm.lib()
    f = L.pqm_dequantize
    assert f(7, A16, A16, None, 4, 32, 1, A16, None) == 4
    assert f(1, A16, A16, None, 4, 48, 1, A16, None) == 2
    assert f(2, A16, A16, None, 4, 32, 1, A16, None) == 1          # no s_outer
    assert f(2, A16, A16, A16, 4, 24, 1, A16, None) == 2
    assert f(1, A16, A16, None, 4, 32, 1, BAD, None) == 3
    assert f(1, A16, A16, None, 0, 32, 1, None, None) == 0         # empty: no-op


def test_quantize_fp8_block_validation():
    L = pqm.lib()
    f = L.pqm_quantize_fp8_block
    assert f(A16, 64, 256, 256, 2, A16, A16, None) == 2        # block rows 1 or 128
    assert f(A16, 64, 192, 192, 1, A16, A16, None) == 2        # cols % 128
    assert f(A16, 64, 256, 256, 128, A16, A16, None) == 2      # rows % 128
    assert f(A16, 64, 256, 128, 1, A16, A16, None) == 2        # ld < cols
    assert f(None, 64, 256, 256, 1, A16, A16, None) == 1
    assert f(A16, 64, 256, 256, 1, A16, None, None) == 1
    assert f(BAD, 64, 256, 256, 1, A16, A16, None) == 3
    assert f(A16, 64, 256, 256, 1, A16, BAD, None) == 3
    assert f(A16, 0, 256, 256, 1, None, None, None) == 0       # empty: no-op


def test_grouped_gemm_validation():
    L = pqm.lib()
    f = L.pqm_moe_grouped_gemm
    args = lambda **kw: [kw.get("fmt", 1), kw.get("kind", 0), A16, A16, None, A16, A16, None,
                         kw.get("brps", 0), kw.get("bias"), A16, kw.get("G", 4), kw.get("M", 64),
                         64, kw.get("K", 64), A16, kw.get("out", 1), None, 0, None]
    assert f(*args(fmt=5)) == 4
    assert f(*args(kind=9)) == 4
    assert f(*args(out=3)) == 4
    assert f(*args(fmt=3, kind=1)) == 4             # block FP8: forward only
    assert f(*args(fmt=3, K=64)) == 2               # block FP8: K % 128
    assert f(*args(fmt=3, K=128)) == 2              # block FP8: N % 128 (N = 64)
    assert f(*args(fmt=2, kind=1)) == 4             # NVFP4: forward only
    assert f(*args(fmt=2, kind=2)) == 4
    assert f(*args(kind=1)) == 2                    # MXFP8 dgrad: K % 128
    assert f(*args(kind=1, K=4096)) == 2            # MXFP8 dgrad: K <= 2048
    assert f(*args(kind=2, M=48)) == 2              # MXFP8 wgrad: M_total % 32
    assert f(*args(kind=2, M=1 << 24)) == 2         # MXFP8 wgrad: 32-bit panel offsets
    a = args()
    a[3] = BAD                                      # MXFP8 scales 4-byte aligned
    assert f(*a) == 3
    assert f(*args(K=48)) == 2
    assert f(*args(fmt=2, K=40)) == 2
    assert f(*args(fmt=2, brps=3)) == 2
    assert f(*args(fmt=0, K=12)) == 2
    assert f(*args(G=-1)) == 2
    assert f(*args(G=0)) == 0                       # nothing to do
    a = args()
    a[2] = BAD
    assert f(*a) == 3
    assert f(*args(kind=1, K=128, bias=A16)) == 4   # bias: forward only
    assert f(*args(kind=2, bias=A16)) == 4
    assert f(*args(bias=ctypes.c_void_p(0x10002))) == 3  # bias 4-byte aligned
    assert f(*args(G=0, bias=A16)) == 0


def test_grouped_gemm_workspace_size():
    """Only the MXFP8 weight gradient takes a workspace (its tile counter);
    the query is host-only."""
    ws = pqm.lib().pqm_moe_grouped_gemm_workspace_size
    assert ws(1, 2) == 4
    for fmt in (0, 1, 2, 3):
        for kind in (0, 1, 2):
            if (fmt, kind) != (1, 2):
                assert ws(fmt, kind) == 0


def test_validate_offsets_arguments():
    f = pqm.lib().pqm_validate_offsets
    assert f(A16, -1, 10, 1, A16, None) == 2
    assert f(A16, 3, -1, 1, A16, None) == 2
    assert f(A16, 3, 10, 0, A16, None) == 2
    assert f(None, 3, 10, 1, A16, None) == 1
    assert f(A16, 3, 10, 1, None, None) == 1
    assert f(BAD, 3, 10, 1, A16, None) == 3
    assert f(A16, 3, 10, 1, BAD, None) == 3


def test_fc2_online_nvfp4_arguments():
    """Argument errors of pqm_moe_fc2_online_nvfp4 come back before any
    launch (p, w_q, w_scale, w_outer, rps, offsets, G, M, N, K, out, dtype,
    gs_out, q_out, sb_out, stream)."""
    f = pqm.lib().pqm_moe_fc2_online_nvfp4
    ok = [A16, A16, A16, A16, 64, A16, 2, 100, 64, 512, A16, 0, A16, A16, A16, None]

    def call(**kw):
        a = list(ok)
        for i, v in kw.items():
            a[int(i[1:])] = v
        return f(*a)
    assert call(a11=2) == 4                      # out dtype
    assert call(a9=384) == 2                     # K % 256
    assert call(a9=0) == 2                       # empty contraction
    assert call(a7=-1) == 2
    assert call(a4=0) == 2                       # rows per scale >= 1
    assert call(a4=3) == 2                       # G * N % rps
    assert call(a0=None) == 1
    assert call(a3=None) == 1                    # outer scales
    assert call(a10=None) == 1                   # out
    assert call(a14=None) == 1                   # q_out without sb_out
    assert call(a0=BAD) == 3
    assert call(a2=ctypes.c_void_p(0x10001)) == 3  # w_scale 4-byte
    assert call(a13=BAD) == 3                    # q_out 16-byte
    assert call(a12=ctypes.c_void_p(0x10001)) == 3  # gs_out 4-byte
    assert call(a6=0) == 0 and call(a7=0) == 0 and call(a8=0) == 0  # nothing to do


def test_fc2_online_nvfp4_split_arguments():
    """Argument errors of pqm_moe_fc2_online_nvfp4_split come back before any
    launch (p, w_q, w_scale, w_outer, rps, offsets, G, M, N, K, out, dtype,
    gs_out, q_out, sb_out, ratio_out, stream): every buffer is required, K is
    at most 4096 (the ratios of a tile row held in LDS)."""
    f = pqm.lib().pqm_moe_fc2_online_nvfp4_split
    ok = [A16, A16, A16, A16, 64, A16, 2, 100, 64, 512, A16, 0, A16, A16, A16, A16, None]

    def call(**kw):
        a = list(ok)
        for i, v in kw.items():
            a[int(i[1:])] = v
        return f(*a)
    assert call(a11=2) == 4                      # out dtype
    assert call(a9=384) == 2                     # K % 256
    assert call(a9=4096 + 256) == 2              # K above 4096
    assert call(a9=0) == 2
    assert call(a4=3) == 2                       # G * N % rps
    for i in (0, 1, 2, 3, 5, 10, 12, 13, 14, 15):  # every buffer is required
        assert call(**{f"a{i}": None}) == 1, i
    assert call(a13=BAD) == 3                    # q_out 16-byte
    assert call(a14=ctypes.c_void_p(0x10001)) == 3  # sb_out 4-byte
    assert call(a15=ctypes.c_void_p(0x10002)) == 3  # ratio_out 4-byte
    assert call(a6=0) == 0 and call(a7=0) == 0 and call(a8=0) == 0  # nothing to do


def test_glue_validation():
    L = pqm.lib()
    assert L.pqm_moe_route(A16, 8, 0, 4, 0, A16, A16, A16, A16, A16, 1 << 20, None) == 2
    assert L.pqm_moe_route(A16, 8, 2, 5000, 0, A16, A16, A16, A16, A16, 1 << 20, None) == 2
    assert L.pqm_moe_route(A16, 8, 2, 4, 0, A16, A16, A16, A16, A16, 0, None) == 5
    assert L.pqm_moe_route(A16, 8, 2, 4, 3, A16, A16, A16, A16, A16, 1 << 20, None) == 4
    assert L.pqm_moe_route(A16, 8, 2, 4, 1, A16, A16, None, A16, A16, 1 << 20, None) == 1
    # one int32 count per expert per 256 assignments, then one int64 total per expert
    assert L.pqm_moe_route_workspace(8192, 8, 128) == 256 * 128 * 4 + 128 * 8
    assert L.pqm_moe_route_workspace(0, 8, 128) == 0
    assert L.pqm_moe_gather_rows(A16, 4, 16, A16, 4, 0, A16, None) == 2
    f = L.pqm_moe_pad_rows
    assert f(A16, 64, 128, A16, 4, 0, A16, A16, 200, None) == 2      # align >= 1
    assert f(A16, 64, 24, A16, 4, 32, A16, A16, 200, None) == 2      # row_bytes % 16
    assert f(A16, 64, 128, A16, 4, 32, A16, A16, 187, None) == 2     # < 64 + 4 * 31 rows
    assert f(A16, 64, 128, None, 4, 32, A16, A16, 188, None) == 1
    assert f(A16, 64, 128, A16, 4, 32, None, A16, 188, None) == 1
    assert f(BAD, 64, 128, A16, 4, 32, A16, A16, 188, None) == 3
    assert f(A16, 64, 128, A16, 4, 32, BAD, A16, 188, None) == 3
    assert L.pqm_swiglu_prob(A16, A16, None, 4, 12, A16, None) == 2
    assert L.pqm_swiglu_prob(BAD, A16, None, 4, 16, A16, None) == 3
    f = L.pqm_swiglu_prob_quantize_mxfp8
    assert f(A16, A16, None, 4, 48, None, A16, A16, None) == 2       # inter % 32
    assert f(A16, A16, None, 4, 64, None, None, A16, None) == 1      # q
    assert f(A16, None, None, 4, 64, None, A16, A16, None) == 1      # prob
    assert f(BAD, A16, None, 4, 64, None, A16, A16, None) == 3
    assert f(A16, A16, None, 4, 64, BAD, A16, A16, None) == 3        # d misaligned
    assert f(A16, A16, None, 0, 64, None, None, None, None) == 0     # empty
    g = L.pqm_moe_gemm_swiglu_quantize_mxfp8
    ok = (A16, A16, A16, A16, A16, 4, 64, 128, 256, A16, None, A16, A16, None)
    assert g(*ok[:7], 96, *ok[8:]) == 2                               # inter % 128
    assert g(*ok[:8], 4096, *ok[9:]) == 2                             # K > 2048
    assert g(*ok[:8], 200, *ok[9:]) == 2                              # K % 128
    assert g(*ok[:11], None, *ok[12:]) == 1                           # q
    assert g(*ok[:11], BAD, *ok[12:]) == 3                            # q misaligned
    assert g(BAD, *ok[1:]) == 3
    assert L.pqm_moe_combine(A16, A16, None, 4, 0, 16, A16, None) == 2
    assert L.pqm_moe_combine(A16, None, None, 4, 2, 16, A16, None) == 1


def test_route_noalloc_validation():
    """The no-allocation routing entry point rejects inputs whose counts do
    not fit its fixed scratch array before anything is enqueued."""
    L = pqm.lib()
    f = L.pqm_moe_route_noalloc
    limit = 4 << 20
    assert L.pqm_moe_route_workspace(65536, 8, 256) <= limit
    assert L.pqm_moe_route_workspace(1 << 20, 8, 4096) > limit
    assert f(A16, 1 << 20, 8, 4096, 0, A16, A16, A16, A16, None) == 5
    assert f(A16, 64, 8, 4097, 0, A16, A16, A16, A16, None) == 2
    assert f(A16, 64, 8, 16, 2, A16, A16, A16, A16, None) == 4
    assert f(A16, 64, 8, 16, 0, None, A16, A16, A16, None) == 1
    assert f(None, 64, 8, 16, 0, A16, A16, A16, A16, None) == 1
    assert f(A16, 64, 8, 16, 0, BAD, A16, A16, A16, None) == 3


def test_swiglu_quantize_nvfp4_validation():
    L = pqm.lib()
    f = L.pqm_swiglu_prob_quantize_nvfp4
    assert f(A16, A16, None, 64, 40, None, A16, A16, A16, None) == 2       # inter % 16
    assert f(A16, A16, None, 64, 1 << 15, None, A16, A16, A16, None) == 2  # inter > 16384
    assert f(None, A16, None, 64, 64, None, A16, A16, A16, None) == 1
    assert f(A16, A16, None, 64, 64, None, A16, None, A16, None) == 1
    assert f(BAD, A16, None, 64, 64, None, A16, A16, A16, None) == 3
    assert f(A16, A16, None, 64, 64, BAD, A16, A16, A16, None) == 3
    assert f(A16, A16, None, 0, 64, None, None, None, None, None) == 0   # nothing to do
