"""Brute-force nearest-grid search in exact rational arithmetic.

Independent of the oracle: no binary search, no midpoint products, no
binary64.  Every grid value is built as a Fraction from the format's bit
fields, and rounding is an argmin of |grid - v| over the whole grid, with
ties broken toward the even code.  Slow; used on small inputs only.
"""
from __future__ import annotations

from fractions import Fraction as Fr

import numpy as np


def _e4m3(c: int) -> Fr:
    e, m = (c >> 3) & 15, c & 7
    if e == 0:
        return Fr(m, 512)
    return (8 + m) * Fr(2) ** (e - 10)


E4M3 = [_e4m3(c) for c in range(127)]          # 0x7F is NaN: excluded
E2M1 = [Fr(0), Fr(1, 2), Fr(1), Fr(3, 2), Fr(2), Fr(3), Fr(4), Fr(6)]


def nearest(grid, v: Fr) -> int:
    """Code of the grid point nearest |v|, ties to the even code; beyond the
    top the nearest point is the top (saturation)."""
    a = abs(v)
    best = None
    for c, g in enumerate(grid):
        d = abs(g - a)
        key = (d, c % 2)
        if best is None or key < best[0]:
            best = (key, c)
    return best[1]


def bf16_value(bits: int) -> Fr:
    bits &= 0xFFFF
    sign = -1 if bits & 0x8000 else 1
    e, m = (bits >> 7) & 0xFF, bits & 0x7F
    assert e != 0xFF, "finite only"
    if e == 0:
        return sign * Fr(m) * Fr(2) ** -133
    return sign * Fr(128 + m) * Fr(2) ** (e - 134)


def _round_binary(v: Fr, mant_bits: int, emin: int, emax: int):
    """Nearest binary float with mant_bits explicit mantissa bits, minimum
    normal exponent emin, max exponent emax; ties to even; returns a Fraction
    or None for overflow."""
    if v == 0:
        return Fr(0)
    a = abs(v)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fr(2) ** e > a:
        e -= 1
    e = max(e, emin)
    q = Fr(2) ** (e - mant_bits)
    n = a / q
    lo = n.numerator // n.denominator
    rem = n - lo
    if rem > Fr(1, 2) or (rem == Fr(1, 2) and lo % 2 == 1):
        lo += 1
    r = lo * q
    top = (2 - Fr(2) ** -mant_bits) * Fr(2) ** emax
    if r > top:
        return None
    return r if v > 0 else -r


def round_fp32(v: Fr):
    return _round_binary(v, 23, -126, 127)


def round_bf16(v: Fr):
    return _round_binary(v, 7, -126, 127)


def fr_to_bf16_bits(v) -> int:
    """Fraction (exactly a bf16 value) or None (overflow) -> bits."""
    if v is None:
        return 0x7F80
    f = np.array([float(v)], np.float32)
    return int((f.view(np.uint32)[0] >> 16) & 0xFFFF)


def mx_scale_exponent(a: Fr) -> int:
    """Smallest e in [-127, 127] with a <= 448 * 2^e."""
    return min(e for e in range(-127, 128) if a <= 448 * Fr(2) ** e)


def mxfp8_block(xbits):
    """One 32-element block: (codes, scale byte)."""
    vals = [bf16_value(int(b)) for b in xbits]
    a = max(abs(v) for v in vals)
    e = mx_scale_exponent(a)
    sc = Fr(2) ** e
    codes = []
    for v, b in zip(vals, xbits):
        c = nearest(E4M3, v / sc)
        codes.append(c | (0x80 if int(b) & 0x8000 else 0))
    return codes, e + 127


def nvfp4(xbits: np.ndarray, rows_per_group: int = 1):
    """Whole NVFP4 quantizer in Fractions: returns (q bytes, sb, sg)."""
    R, C = xbits.shape
    G = R // rows_per_group
    q = np.zeros((R, C // 2), np.uint8)
    sb = np.zeros((R, C // 16), np.uint8)
    sg = np.zeros(G, np.float32)
    for g in range(G):
        rows = range(g * rows_per_group, (g + 1) * rows_per_group)
        A = max(abs(bf16_value(int(b))) for r in rows for b in xbits[r])
        s_g = round_fp32(A / 2688)
        sg[g] = np.float32(float(s_g))
        for r in rows:
            q[r], sb[r] = nvfp4_row_given_scale(xbits[r], s_g)
    return q, sb, sg


def nvfp4_row_given_scale(xbits_row, s_g: Fr):
    """NVFP4 blocks of one row under the outer scale s_g (a Fraction):
    returns (q bytes [C/2], sb [C/16])."""
    C = len(xbits_row)
    q = np.zeros(C // 2, np.uint8)
    sb = np.zeros(C // 16, np.uint8)
    for blk in range(C // 16):
        bits = [int(b) for b in xbits_row[blk * 16:(blk + 1) * 16]]
        vals = [bf16_value(b) for b in bits]
        ab = max(abs(v) for v in vals)
        c_sb = 0 if s_g == 0 else nearest(E4M3, ab / (6 * s_g))
        sb[blk] = c_sb
        nib = []
        for v, b in zip(vals, bits):
            sign = 8 if b & 0x8000 else 0
            if c_sb == 0:
                nib.append(sign)
            else:
                nib.append(sign | nearest(E2M1, v / (E4M3[c_sb] * s_g)))
        for j in range(8):
            q[blk * 8 + j] = nib[2 * j] | (nib[2 * j + 1] << 4)
    return q, sb


def nvfp4_values(q_row, sb_row, s_g: Fr):
    """Exact decoded values q * s_b * s_g of one row, as Fractions."""
    out = []
    for i in range(2 * len(q_row)):
        nib = (int(q_row[i // 2]) >> (4 * (i % 2))) & 0xF
        v = E2M1[nib & 7] * E4M3[int(sb_row[i // 16]) & 0x7F] * s_g
        out.append(-v if nib & 8 else v)
    return out


def fp8_block(xbits: np.ndarray, block_rows: int):
    """Block-scaled FP8 in Fractions: s = binary32(A / 448) per block of
    block_rows x 128, codes = nearest E4M3 of x / s (sign kept, s = 0 gives
    signed zeros).  Returns (q bytes, s float32)."""
    R, C = xbits.shape
    q = np.zeros((R, C), np.uint8)
    s = np.zeros((R // block_rows, C // 128), np.float32)
    for rb in range(R // block_rows):
        for cb in range(C // 128):
            rows = range(rb * block_rows, (rb + 1) * block_rows)
            cols = range(cb * 128, (cb + 1) * 128)
            A = max(abs(bf16_value(int(xbits[r, c]))) for r in rows for c in cols)
            sc = round_fp32(A / 448)
            s[rb, cb] = np.float32(float(sc))
            for r in rows:
                for c in cols:
                    b = int(xbits[r, c])
                    sign = 0x80 if b & 0x8000 else 0
                    q[r, c] = sign if sc == 0 else sign | nearest(E4M3, bf16_value(b) / sc)
    return q, s
