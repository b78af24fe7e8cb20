"""Pins of the oracle's online amax compensation loop and its two-pass
counterpart ([MT] "miniTE technical report", 5.6).  CPU only.

The pins reach the loop from outside its own code:
* a hand-derived worked example (tests/golden/online_amax_example.txt);
* a replay of the loop in exact rational arithmetic on tiny inputs, with the
  encodings taken by the brute-force nearest-grid search;
* the closed form O_final gs_final = sum_i gs_i dO_i (a wrong rescale
  direction, a missed rescale or a wrong final factor breaks it);
* reductions to the pinned per-token quantizer: the given-scale encoding
  equals the per-token encoding of the row with its running maximum appended,
  a single K-tile is the two-pass path, and so is any row whose maximum lies
  in its first non-zero tile;
* all-zero rows give zero, and zero leading tiles are skipped."""
from __future__ import annotations

import os
from fractions import Fraction as Fr

import numpy as np
import pytest

import bruteforce as bf
import oracle
from precision_quantization_moe_amd import workloads as wl

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "online_amax_example.txt")


def _bits(vals) -> np.ndarray:
    v = np.asarray(vals, np.float32)
    b = wl.f32_to_bf16_bits(v)
    assert np.array_equal(oracle.bf16_to_f64(b), v.astype(np.float64)), "exact in bf16"
    return b


def _parse(spec: str):
    out = []
    for tok in spec.split(","):
        tok = tok.strip()
        n = 1
        if "*" in tok:
            n_s, tok = tok.split("*")
            n = int(n_s)
        out.extend([tok] * n)
    return out


def _golden():
    kv = {}
    with open(GOLDEN) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                k, v = [p.strip() for p in line.split("|")]
                kv[k] = v
    return kv


def _w2(rng, N, I, scale=0.05):
    w = oracle.f64_to_bf16(rng.standard_normal((N, I)) * scale)
    q, sb, sg = oracle.quantize_nvfp4(w, rows_per_group=N)
    return q, sb, float(sg[0])


def _p(rng, R, I, spread=True):
    """Weighted SwiGLU rows in bf16; with spread, the row maxima land in
    varied tiles (a ramp of magnitudes along the row)."""
    c = rng.standard_normal((R, 2 * I))
    if spread:
        c[:, :I] *= rng.uniform(0.2, 3.0, (R, 1)) * np.linspace(0.3, 2.0, I)[None, :] \
            ** rng.uniform(-2, 2, (R, 1))
    return oracle.f64_to_bf16(oracle.swiglu_prob(c, rng.uniform(0.05, 1.0, R)))


# ------------------------------------------------------------ worked example

def test_online_amax_worked_example():
    g = _golden()
    p = _bits([float(t) for t in _parse(g["p"])])[None, :]
    w = _bits([float(t) for t in _parse(g["w2"])])[None, :]
    w2q, w2sb, w2sg = oracle.quantize_nvfp4(w, rows_per_group=1)
    assert int(w2sg.view(np.uint32)[0]) == int(g["w2_sg"], 16)
    tile = int(g["tile"])
    y, rec = oracle.online_amax_fc2(p, tile, w2q, w2sb, float(w2sg[0]))
    assert rec["gs"][0].view(np.uint32).tolist() == [int(t, 16) for t in _parse(g["online_gs"])]
    assert rec["sb"][0].tolist() == [int(t, 16) for t in _parse(g["online_sb"])]
    assert rec["q"][0].tolist() == [int(t, 16) for t in _parse(g["online_q"])]
    assert y[0, 0] == float(g["online_y"])
    y2, (q2, sb2, sg2) = oracle.two_pass_fc2(p, w2q, w2sb, float(w2sg[0]))
    assert sb2[0].tolist() == [int(t, 16) for t in _parse(g["two_sb"])]
    assert q2[0].tolist() == [int(t, 16) for t in _parse(g["two_q"])]
    assert int(sg2.view(np.uint32)[0]) == int(g["two_sg"], 16)
    assert y2[0, 0] == float(g["two_y"])
    rep = oracle.online_amax_report(p, tile, w2q, w2sb, float(w2sg[0]))
    assert Fr(rep["blocks_changed"]).limit_denominator(100) == Fr(g["blocks_changed"])
    assert rep["comp_rel_fp64"] == 0.0 and rep["comp_rel_fp32"] == 0.0


# ------------------------------------------------- exact rational replay

def _fraction_loop(p_bits, tile, w2q, w2sb, w2sg):
    """The loop in Fractions with brute-force encodings: per row, returns
    (Y as Fractions [N], gs per tile as Fractions, q bytes, sb bytes)."""
    R, I = p_bits.shape
    N = w2q.shape[0]
    w2 = [bf.nvfp4_values(w2q[n], w2sb[n], Fr(1)) for n in range(N)]
    out = []
    for r in range(R):
        gamax, gs_prev = Fr(0), Fr(0)
        O = [Fr(0)] * N
        gs_list, q_row, sb_row = [], [], []
        for i in range(I // tile):
            seg = p_bits[r, i * tile:(i + 1) * tile]
            gamax = max(gamax, max(abs(bf.bf16_value(int(b))) for b in seg))
            if gamax == 0:
                gs_list.append(Fr(0))
                q_row += [0] * (tile // 2)
                sb_row += [0] * (tile // 16)
                continue
            gs = bf.round_fp32(gamax / 2688)
            q, sb = bf.nvfp4_row_given_scale(seg, gs)
            vals = bf.nvfp4_values(q, sb, Fr(1))
            for n in range(N):
                d = sum(v * w for v, w in zip(vals, w2[n][i * tile:(i + 1) * tile]))
                O[n] = O[n] * (gs_prev / gs) + d
            gs_prev = gs
            gs_list.append(gs)
            q_row += q.tolist()
            sb_row += sb.tolist()
        Y = [o * gs_prev * Fr(float(np.float32(w2sg))) for o in O]
        out.append((Y, gs_list, q_row, sb_row))
    return out


@pytest.mark.parametrize("seed", range(3))
def test_online_loop_vs_fraction_replay(seed):
    rng = np.random.Generator(np.random.PCG64(70 + seed))
    R, I, N, tile = 3, 64, 4, 16
    p = _p(rng, R, I)
    p[0, :16] = 0                                   # a skipped leading tile
    w2q, w2sb, w2sg = _w2(rng, N, I)
    y, rec = oracle.online_amax_fc2(p, tile, w2q, w2sb, w2sg)
    for r, (Y, gs_list, q_row, sb_row) in enumerate(_fraction_loop(p, tile, w2q, w2sb, w2sg)):
        assert rec["q"][r].tolist() == q_row
        assert rec["sb"][r].tolist() == sb_row
        assert [Fr(float(g)) for g in rec["gs"][r]] == gs_list
        ref = np.array([float(v) for v in Y])
        assert np.allclose(y[r], ref, rtol=1e-13, atol=1e-13 * np.abs(ref).max())


# --------------------------------------------------------------- closed form

def test_online_telescoped_sum():
    """O_n gs_n = sum_i gs_i dO_i, so Y = gs_W2 sum_i gs_i dO_i with dO_i
    formed from the recorded encodings; a binary32 accumulator stays within a
    few binary32 roundings of it per tile."""
    rng = np.random.Generator(np.random.PCG64(81))
    R, I, N, tile = 16, 512, 24, 64
    p = _p(rng, R, I)
    w2q, w2sb, w2sg = _w2(rng, N, I)
    w2 = oracle.decode_nvfp4(w2q, w2sb, np.ones(1, np.float32), rows_per_group=N)
    y, rec = oracle.online_amax_fc2(p, tile, w2q, w2sb, w2sg)
    vals = oracle.decode_nvfp4(rec["q"], rec["sb"], np.ones(R, np.float32))
    want = np.zeros((R, N))
    for i in range(I // tile):
        sl = slice(i * tile, (i + 1) * tile)
        want += rec["gs"][:, i:i + 1].astype(np.float64) * (vals[:, sl] @ w2[:, sl].T)
    want *= float(np.float32(w2sg))
    scale = np.abs(want).max(axis=1, keepdims=True)
    assert np.all(np.abs(y - want) <= 1e-13 * scale)
    # the running scale never decreases along the row
    gs = rec["gs"]
    for r in range(R):
        nz = gs[r][gs[r] > 0]
        assert np.all(np.diff(nz) >= 0)
    y32, _ = oracle.online_amax_fc2(p, tile, w2q, w2sb, w2sg, np.float32)
    assert np.all(np.abs(y32 - want) <= 4 * (I // tile) * 2.0 ** -24 * np.abs(
        vals @ w2.T * rec["gs"].max(axis=1, keepdims=True) * float(np.float32(w2sg))).max()
        + 1e-6 * scale)


# ------------------------------------------ reductions to the pinned quantizer

def test_given_scale_is_per_token_of_row_with_its_running_max():
    """Encoding a tile under gs = fp32(m / 2688) for any m >= the tile's max
    equals the per-token encoding of the tile with one more block holding m."""
    rng = np.random.Generator(np.random.PCG64(82))
    R, C = 32, 64
    x = oracle.f64_to_bf16(rng.standard_normal((R, C)) * rng.uniform(1e-3, 10, (R, 1)))
    xa = np.abs(oracle.bf16_to_f64(x)).max(axis=1)
    m = oracle.f64_to_bf16((xa * rng.uniform(1.0, 40.0, R))[:, None])[:, 0]
    m = np.maximum(m, oracle.f64_to_bf16(xa[:, None])[:, 0])      # >= row max
    ext = np.concatenate([x, np.zeros((R, 16), np.uint16)], axis=1)
    ext[:, C] = m
    q1, sb1, sg1 = oracle.quantize_nvfp4(ext)
    q2, sb2 = oracle.quantize_nvfp4_given_scale(x, sg1)
    assert np.array_equal(q2, q1[:, :C // 2]) and np.array_equal(sb2, sb1[:, :C // 16])
    # and against the brute-force search for a few rows
    for r in range(4):
        bq, bsb = bf.nvfp4_row_given_scale(x[r], Fr(float(sg1[r])))
        assert np.array_equal(bq, q2[r]) and np.array_equal(bsb, sb2[r])


def test_single_tile_is_two_pass():
    rng = np.random.Generator(np.random.PCG64(83))
    R, I, N = 12, 256, 16
    p = _p(rng, R, I)
    w2q, w2sb, w2sg = _w2(rng, N, I)
    y, rec = oracle.online_amax_fc2(p, I, w2q, w2sb, w2sg)
    y2, (q2, sb2, sg2) = oracle.two_pass_fc2(p, w2q, w2sb, w2sg)
    assert np.array_equal(rec["q"], q2) and np.array_equal(rec["sb"], sb2)
    assert np.array_equal(rec["gs"][:, 0], sg2)
    assert np.allclose(y, y2, rtol=1e-13, atol=0)


def test_max_in_first_nonzero_tile_is_two_pass():
    """Rows whose maximum lies in the first non-zero tile: every tile is
    encoded under the final outer scale, so bytes and Y equal the two-pass
    path; other rows have gs growing and at least one tile encoded early."""
    rng = np.random.Generator(np.random.PCG64(84))
    R, I, N, tile = 10, 256, 8, 32
    p = oracle.f64_to_bf16(rng.standard_normal((R, I)))
    p[:, 0] = 0x4120                                   # 10.0 > any N(0,1) draw here
    p[2, :tile] = 0                                    # leading zero tile
    p[2, tile] = 0x4120
    w2q, w2sb, w2sg = _w2(rng, N, I)
    y, rec = oracle.online_amax_fc2(p, tile, w2q, w2sb, w2sg)
    y2, (q2, sb2, sg2) = oracle.two_pass_fc2(p, w2q, w2sb, w2sg)
    assert np.array_equal(rec["q"], q2) and np.array_equal(rec["sb"], sb2)
    assert np.allclose(y, y2, rtol=1e-13, atol=1e-15)
    assert rec["gs"][2, 0] == 0 and np.all(rec["gs"][2, 1:] == sg2[2])
    # a row whose maximum sits in its last tile: earlier tiles encoded early
    p[4, 0] = 0x3F80                                   # 1.0
    p[4, I - 1] = 0x4120
    y, rec = oracle.online_amax_fc2(p, tile, w2q, w2sb, w2sg)
    assert rec["gs"][4, 0] < rec["gs"][4, -1] == oracle.quantize_nvfp4(p[4:5])[2][0]


def test_zero_rows_output_zero():
    rng = np.random.Generator(np.random.PCG64(85))
    R, I, N, tile = 4, 128, 8, 32
    p = _p(rng, R, I)
    p[1] = 0
    p[3] = 0x8000                                      # negative zeros
    w2q, w2sb, w2sg = _w2(rng, N, I)
    y, rec = oracle.online_amax_fc2(p, tile, w2q, w2sb, w2sg)
    for r in (1, 3):
        assert np.all(y[r] == 0) and np.all(rec["gs"][r] == 0) and np.all(rec["sb"][r] == 0)
    assert np.all(np.abs(y[[0, 2]]).max(axis=1) > 0)


def test_report_fields_in_range():
    """The report on a workload-like row mix: the binary64 loop compensates
    exactly up to rounding, a binary32 accumulator to about 2^-24 per tile,
    and the early encodings move the result by much less than the format's
    own error against the unquantized product."""
    rng = np.random.Generator(np.random.PCG64(86))
    R, I, N, tile = 32, 512, 32, 64
    p = _p(rng, R, I)
    w2q, w2sb, w2sg = _w2(rng, N, I)
    rep = oracle.online_amax_report(p, tile, w2q, w2sb, w2sg)
    assert rep["comp_rel_fp64"] < 1e-14
    assert rep["comp_rel_fp32"] < 1e-6
    assert 0 < rep["blocks_changed"] < 1
    assert rep["rel_vs_two_pass_max"] < 0.2
    assert rep["rel_two_pass_vs_exact"] < 0.2 and rep["rel_online_vs_exact"] < 0.2
