"""GPU parity of the online-amax NVFP4 down projection
(pqm_moe_fc2_online_nvfp4 and its split form
pqm_moe_fc2_online_nvfp4_split, [MT] "miniTE technical report", 5.6) against
the oracle's loop (oracle.online_amax_fc2, 128-wide K-tiles).

Bars:
  * the codes and block scales P was encoded with, tile by tile, and each
    row's final outer scale: bit-exact (quantized decisions, both sides
    exact);
  * Y: relative L2 <= 1e-3 per row on binary32 output against the oracle's
    binary64 loop (the kernel accumulates in binary32 and moves the
    accumulator by a binary32 gs_prev / gs), plus one bf16 rounding (2^-8)
    for bf16 output;
  * split form: each tile's stored gs_prev / gs bit-exact against one
    binary32 division of the oracle's per-tile gs, and Y, gs, codes and
    block scales bit for bit those of the one-kernel path.

W2 is quantized with one outer scale per expert tensor (or per scope of
w_rows_per_scale rows) by the library's per-token quantizer on the device and
by the oracle's on the host, from the same bf16 bytes (their byte equality is
established separately)."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import precision_quantization_moe_amd as pqm
from precision_quantization_moe_amd import workloads as wl
from gpu_util import assert_bytes_equal, dev, dev_bf16, host, host_u16, requires_gpu

pytestmark = [pytest.mark.gpu, requires_gpu]

TOL = 1e-3
TILE = 128


def _offsets(sizes):
    return np.concatenate([[0], np.cumsum(sizes)]).astype(np.int64)


def _rel_rows(got, want):
    num = np.linalg.norm(got.astype(np.float64) - want, axis=1)
    den = np.linalg.norm(want, axis=1)
    return np.where(den > 0, num / np.where(den > 0, den, 1), num)


def _p_rows(rng, R, I):
    """Weighted SwiGLU rows (bf16 bits) whose maxima arrive in varied tiles:
    a ramp of gate magnitudes along the row with a per-row exponent, some
    rows with leading zero tiles, a late burst, or all zeros (signed)."""
    c = rng.standard_normal((R, 2 * I))
    c[:, :I] *= rng.uniform(0.2, 3.0, (R, 1)) * np.linspace(0.3, 2.0, I)[None, :] \
        ** rng.uniform(-2, 2, (R, 1))
    p = oracle.swiglu_prob(c, rng.uniform(0.05, 1.0, R))
    r = np.arange(R)
    p[r % 5 == 1, :TILE] = 0.0                      # first tile skipped
    p[r % 7 == 2, :2 * TILE] = 0.0                  # two leading zero tiles
    p[r % 3 == 0, -TILE:] *= 8.0                    # maximum in the last tile
    bits = oracle.f64_to_bf16(p)
    bits[r % 11 == 4] = np.where(rng.random((int((r % 11 == 4).sum()), I)) < 0.5,
                                 0x8000, 0x0000)   # all-zero rows, signed zeros
    return bits


def _want_ratio(gs_rec):
    """Each tile's gs_prev / gs from the oracle's per-tile gs (0 while the
    row's maximum is zero): one binary32 division, 1 for a skipped tile."""
    prev = np.concatenate([np.zeros((gs_rec.shape[0], 1), np.float32), gs_rec[:, :-1]], axis=1)
    with np.errstate(invalid="ignore", divide="ignore"):
        q = prev / gs_rec
    return np.where(gs_rec > 0, q, np.float32(1.0)).astype(np.float32)


def _case(sizes, N, K, seed, out_dtype=pqm.OUT_FP32, rps=None, split=False):
    """rps: W2 rows per outer scale (default N, one per expert); with rps < N
    the oracle's loop (one W2 scale) runs once per scale scope of W2 rows,
    whose output columns it then fills.  split: the split entry point
    (encode once, then the GEMM with the stored ratios)."""
    rps = rps or N
    rng = np.random.Generator(np.random.PCG64(seed))
    G, M = len(sizes), int(sum(sizes))
    off = _offsets(sizes)
    p = _p_rows(rng, max(M, 1), K)[:M]
    w = wl.normal_bf16((G * N, K), std=0.02, seed=seed + 1)
    qw, sw, gw = pqm.quantize_nvfp4_per_token(dev_bf16(w), rows_per_scale=rps)
    fn = pqm.moe_fc2_online_nvfp4_split if split else pqm.moe_fc2_online_nvfp4
    res = fn(dev_bf16(p), qw, sw, gw, dev(off), N, w_rows_per_scale=rps, out_dtype=out_dtype,
             encodings=True)
    torch.cuda.synchronize()
    y, gs, q, sb = res[:4]
    got_y = host(y.float())
    got = dict(gs=host(gs), q=host(q), sb=host(sb))
    want_y = np.zeros((M, N))
    want = dict(gs=np.zeros(M, np.float32), q=np.zeros((M, K // 2), np.uint8),
                sb=np.zeros((M, K // 16), np.uint8))
    if split:
        got["ratio"] = host(res[4])
        want["ratio"] = np.ones((M, K // TILE), np.float32)
    for g in range(G):
        lo, hi = int(off[g]), int(off[g + 1])
        if hi == lo:
            continue
        for c0 in range(0, N, rps):
            wr = w[g * N + c0:g * N + c0 + rps]
            rq, rsb, rsg = oracle.quantize_nvfp4(wr, rows_per_group=rps)
            yg, rec = oracle.online_amax_fc2(p[lo:hi], TILE, rq, rsb, float(rsg[0]))
            want_y[lo:hi, c0:c0 + rps] = yg
        want["gs"][lo:hi] = rec["gs"].max(axis=1)   # gs only grows; 0 for a zero row
        want["q"][lo:hi] = rec["q"]
        want["sb"][lo:hi] = rec["sb"]
        if split:
            want["ratio"][lo:hi] = _want_ratio(rec["gs"])
    return got_y, got, want_y, want


def _many_small(G, seed):
    sizes = np.random.Generator(np.random.PCG64(seed)).choice([0, 0, 1, 2, 5, 33], size=G)
    sizes[G // 2] = 300
    return sizes.tolist()


@pytest.mark.parametrize("sizes,N,K,rps", [
    ([130, 0, 33, 256, 7, 1], 520, 512, None),   # ragged experts and columns, 4 tiles
    ([300, 129], 256, 768, None),                # 6 tiles, one column tile
    ([64, 200, 0], 200, 256, None),              # 2 tiles (the prologue only), N < one tile
    ([200, 77], 512, 512, 256),                  # W2 scaled per half (gate / up style scopes)
    (_many_small(600, 35), 256, 256, None),      # > 512 experts: the tile lookup's general path
])
@pytest.mark.parametrize("split", [False, True], ids=["one-kernel", "split"])
def test_online_fc2_matches_oracle(sizes, N, K, rps, split):
    got_y, got, want_y, want = _case(sizes, N, K, seed=31 + K, rps=rps, split=split)
    assert_bytes_equal(got["gs"].view(np.uint32), want["gs"].view(np.uint32), "final gs")
    assert_bytes_equal(got["sb"], want["sb"], "block scales")
    assert_bytes_equal(got["q"], want["q"], "codes")
    if split:
        assert_bytes_equal(got["ratio"].view(np.uint32), want["ratio"].view(np.uint32),
                           "per-tile gs_prev / gs")
    r = _rel_rows(got_y, want_y)
    what = sizes if len(sizes) <= 12 else f"{len(sizes)} experts, {sum(sizes)} rows"
    print(f"[online] {what} N={N} K={K} split={split}: max row rel-L2 {r.max():.3e}", flush=True)
    assert r.max() <= TOL, (float(r.max()), int(r.argmax()))
    zero = want["gs"] == 0
    assert zero.any() and not got_y[zero].any()


def test_online_fc2_bf16_out_and_deterministic():
    sizes, N, K = [190, 70], 384, 512
    got_y, _, want_y, _ = _case(sizes, N, K, seed=41, out_dtype=pqm.OUT_BF16)
    r = _rel_rows(got_y, want_y)
    print(f"[online] bf16 out: max row rel-L2 {r.max():.3e}", flush=True)
    assert r.max() <= TOL + 2.0 ** -8
    rng = np.random.Generator(np.random.PCG64(42))
    p = dev_bf16(_p_rows(rng, sum(sizes), K))
    w = wl.normal_bf16((2 * N, K), std=0.02, seed=43)
    qw, sw, gw = pqm.quantize_nvfp4_per_token(dev_bf16(w), rows_per_scale=N)
    off = dev(_offsets(sizes))
    y1, g1 = pqm.moe_fc2_online_nvfp4(p, qw, sw, gw, off, N)
    y2, g2 = pqm.moe_fc2_online_nvfp4(p, qw, sw, gw, off, N)
    torch.cuda.synchronize()
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))
    assert torch.equal(g1, g2)


@pytest.mark.parametrize("sizes,N,K", [([130, 0, 33, 256, 7, 1], 520, 512),
                                         (_many_small(600, 36), 256, 768),
                                         ([1000, 3], 384, 4096)])
def test_online_fc2_split_matches_one_kernel(sizes, N, K):
    """The split entry point against the one-kernel path on the same
    inputs: output (binary32 and bf16), gs, codes and block scales bit for
    bit (the same encoding, accumulation order and epilogue)."""
    rng = np.random.Generator(np.random.PCG64(50 + K))
    G, M = len(sizes), sum(sizes)
    p = dev_bf16(_p_rows(rng, M, K))
    w = wl.normal_bf16((G * N, K), std=0.02, seed=51)
    qw, sw, gw = pqm.quantize_nvfp4_per_token(dev_bf16(w), rows_per_scale=N)
    off = dev(_offsets(sizes))
    for od in (pqm.OUT_FP32, pqm.OUT_BF16):
        a = pqm.moe_fc2_online_nvfp4(p, qw, sw, gw, off, N, out_dtype=od, encodings=True)
        b = pqm.moe_fc2_online_nvfp4_split(p, qw, sw, gw, off, N, out_dtype=od, encodings=True)
        torch.cuda.synchronize()
        for name, x, y in zip(("Y", "gs", "codes", "block scales"), a, b[:4]):
            assert torch.equal(x.view(torch.uint8), y.view(torch.uint8)), (name, od)


def _split_random_cases(n=8, seed=2025):
    """n seeded (sizes, N, K, seed) cases: expert counts 1 to 300 with empty,
    one-row and multi-tile experts, N below, at and across the 256-column
    tile, K from 2 to 32 tiles."""
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        G = int(rng.choice([1, 3, 17, 300]))
        sizes = rng.choice([0, 0, 1, 2, 31, 64, 129, 300], size=G).tolist()
        if sum(sizes) == 0:
            sizes[0] = 7
        N = int(rng.choice([40, 136, 256, 520, 1024]))
        K = int(rng.choice([256, 512, 1024, 2048, 4096]))
        if G * N * K > 4e7 or sum(sizes) * K > 2e7:
            continue
        out.append((sizes, N, K, int(rng.integers(1 << 30))))
    return out


@pytest.mark.parametrize("case", _split_random_cases(),
                         ids=lambda c: f"G{len(c[0])}-M{sum(c[0])}-{c[1]}x{c[2]}")
def test_online_fc2_split_random_shapes(case):
    """The split entry point equals the one-kernel path bit for bit on
    seeded random shapes (both output types, gs, codes, block scales)."""
    sizes, N, K, seed = case
    G, M = len(sizes), sum(sizes)
    print(f"[online] split random G={G} M={M} N={N} K={K}", flush=True)
    rng = np.random.Generator(np.random.PCG64(seed))
    p = dev_bf16(_p_rows(rng, M, K))
    w = wl.normal_bf16((G * N, K), std=0.02, seed=seed + 1)
    qw, sw, gw = pqm.quantize_nvfp4_per_token(dev_bf16(w), rows_per_scale=N)
    off = dev(_offsets(sizes))
    for od in (pqm.OUT_FP32, pqm.OUT_BF16):
        a = pqm.moe_fc2_online_nvfp4(p, qw, sw, gw, off, N, out_dtype=od, encodings=True)
        b = pqm.moe_fc2_online_nvfp4_split(p, qw, sw, gw, off, N, out_dtype=od, encodings=True)
        torch.cuda.synchronize()
        for name, x, y in zip(("Y", "gs", "codes", "block scales"), a, b[:4]):
            assert torch.equal(x.view(torch.uint8), y.view(torch.uint8)), (name, od)


def test_online_fc2_max_in_first_tile_is_two_pass_encoding():
    """Rows whose maximum lies in their first tile are encoded exactly as the
    per-token quantizer encodes the whole row (the two-pass path)."""
    rng = np.random.Generator(np.random.PCG64(44))
    R, N, K = 96, 256, 512
    p = _p_rows(rng, R, K)
    f = oracle.bf16_to_f64(p)
    p[:, 0] = oracle.f64_to_bf16(np.abs(f).max(axis=1) * 1.5)  # the row max up front
    w = wl.normal_bf16((N, K), std=0.02, seed=45)
    qw, sw, gw = pqm.quantize_nvfp4_per_token(dev_bf16(w), rows_per_scale=N)
    pd = dev_bf16(p)
    _, gs, q, sb = pqm.moe_fc2_online_nvfp4(pd, qw, sw, gw, dev(_offsets([R])), N,
                                            encodings=True)
    q2, sb2, sg2 = pqm.quantize_nvfp4_per_token(pd)
    torch.cuda.synchronize()
    assert_bytes_equal(host(q), host(q2), "codes vs per-token")
    assert_bytes_equal(host(sb), host(sb2), "block scales vs per-token")
    assert_bytes_equal(host(gs).view(np.uint32), host(sg2).view(np.uint32), "gs vs per-token")


def test_online_fc2_deepseek_down_full_sampled():
    """DeepSeek-V3 down projection at full size with the online loop: 32768
    routed rows (half uniform, half Zipf over 256 experts) plus the shared
    expert's 4096 rows, N = 7168, K = 2048 (16 tiles), weights [257, 7168,
    2048] N(0, 0.01) drawn on the GPU, one outer scale per expert, bf16
    output.  P: weighted SwiGLU rows generated on the GPU.  Sampled rows of
    sampled experts against the oracle's loop (encodings bit-exact, Y at the
    bar + one bf16 rounding)."""
    T, E, k, H, I = 4096, 256, 8, 7168, 2048
    ids = wl.uniform_plus_zipf_routing(T, E, k)
    off_r, _, _ = oracle.route(ids, E)
    off = np.concatenate([off_r, [T * k + T]]).astype(np.int64)
    M = T * k + T
    gen = torch.Generator(device="cuda").manual_seed(777)
    c = torch.randn(M, 2 * I, generator=gen, device="cuda").to(torch.bfloat16)
    prob = torch.rand(M, generator=gen, device="cuda") * 0.5 + 0.05
    p = pqm.swiglu_prob(c, prob)
    w = (torch.randn((E + 1) * H, I, generator=gen, device="cuda") * 0.01).to(torch.bfloat16)
    qw, sw, gw = pqm.quantize_nvfp4_per_token(w, rows_per_scale=H)
    y, gs, q, sb = pqm.moe_fc2_online_nvfp4(p, qw, sw, gw, dev(off), H, encodings=True)
    y2, gs2, q2, sb2, _ = pqm.moe_fc2_online_nvfp4_split(p, qw, sw, gw, dev(off), H,
                                                         encodings=True)
    torch.cuda.synchronize()
    for name, a, b in (("Y", y, y2), ("gs", gs, gs2), ("codes", q, q2), ("block scales", sb, sb2)):
        assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), f"split {name}"
    del y2, gs2, q2, sb2
    rng = np.random.Generator(np.random.PCG64(46))
    experts = sorted(set(rng.choice(E, 4, replace=False).tolist()) | {0, E - 1, E})
    for e in experts:
        lo, hi = int(off[e]), int(off[e + 1])
        if hi == lo:
            continue
        rows = np.unique(np.concatenate([[lo, hi - 1], rng.integers(lo, hi, 4)]))
        pr = host_u16(p[rows])
        rq, rsb, rsg = oracle.quantize_nvfp4(host_u16(w[e * H:(e + 1) * H]), rows_per_group=H)
        want, rec = oracle.online_amax_fc2(pr, TILE, rq, rsb, float(rsg[0]))
        assert_bytes_equal(host(q[rows]), rec["q"], f"expert {e} codes")
        assert_bytes_equal(host(sb[rows]), rec["sb"], f"expert {e} block scales")
        assert_bytes_equal(host(gs[rows]).view(np.uint32),
                           rec["gs"].max(axis=1).view(np.uint32), f"expert {e} gs")
        r = _rel_rows(oracle.bf16_to_f64(host_u16(y[rows])), want)
        print(f"[online] deepseek fc2 expert {e} ({hi - lo} rows): max row rel-L2 {r.max():.3e}",
              flush=True)
        assert r.max() <= TOL + 2.0 ** -8, (e, float(r.max()))
    del w, qw, c
