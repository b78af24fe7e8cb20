"""Facts about the number formats that the HIP quantizers' binary32 fast paths
rely on, checked exhaustively on the host.

The per-token NVFP4 kernel takes s_b and the element codes from binary32
quotients bracketed by a relative margin, and settles a disagreement between
the bracket ends by the rounding direction of the outer scale s_g = A / 2688.
That is valid because the ideal quotients -- taken with A / 2688 in place of
s_g -- are ratios of short integers, so they are either exactly a rounding
midpoint or far from every midpoint:
  * elements: Q = 2688 x / (s_b A), x and A bf16 (8-bit significands), s_b an
    E4M3 value, against the E2M1 midpoints 0.25 .. 5;
  * block scales: P = 448 a_b / A against the midpoints of consecutive E4M3
    values.
The kernel needs the separation to exceed its bracket width plus the s_g
rounding (about 2^-20 for elements, 2^-19.8 for scales).
"""
import numpy as np


def _e4m3_values():
    vals = []
    for c in range(0, 127):
        e, m = c >> 3, c & 7
        vals.append(m * 2.0 ** -9 if e == 0 else (1 + m / 8) * 2.0 ** (e - 7))
    return np.array(vals)


def _min_separation(ratio, midpoints):
    lr = np.log2(ratio)
    best = 1.0
    for t in midpoints:
        q = ratio * 2.0 ** np.round(np.log2(t) - lr)  # any power-of-two alignment
        rel = np.abs(q - t) / t
        nz = rel[rel > 1e-15]   # exact ties (0) are the cases the direction rule settles
        if nz.size:
            best = min(best, float(nz.min()))
    return best


SIG = np.arange(1, 256, dtype=np.float64)   # bf16 significands, subnormal ones included


def test_e2m1_element_quotients_are_ties_or_far_from_midpoints():
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])
    best = 1.0
    for s in _e4m3_values()[1:]:
        ratio = 2688.0 * SIG[:, None] / (s * SIG[None, :])
        best = min(best, _min_separation(ratio, mids))
    assert best > 2.0 ** -14, best          # 2^-13.81 exhaustively
    assert best > 4 * 2.0 ** -20


def test_e4m3_scale_quotients_are_ties_or_far_from_midpoints():
    v = _e4m3_values()
    mids = (v[1:] + v[:-1]) / 2
    ratio = 448.0 * SIG[:, None] / SIG[None, :]
    best = _min_separation(ratio, mids)
    assert best > 2.0 ** -13, best          # 2^-12.84 exhaustively
    assert best > 4 * 2.0 ** -19.8
