"""Seeded synthetic inputs for the quantizer and MoE expert workloads.

This module holds input generation only (random numbers, routing draws and
the float32 -> bf16 conversion of generated values).  None of the method's
arithmetic is here; both the HIP path and the CPU oracle are fed from it.

The shapes and distributions stand in for the real activations and weights
the pages measure on (Qwen3-30B-A3B and DeepSeek-V3 expert layers; the
datasets and trained weights are not available):

* activations: per-token magnitude m_t ~ LogNormal(0, 1) times N(0, 1)
  entries, with 0.1 % of entries multiplied by 100, placed in 8 fixed
  channels (outlier channels);
* the tiny contract tensor: N(0, 1) with 1 % of entries x50, one all-zero
  row and one row of bf16 max;
* weights: N(0, sigma^2) per expert, drawn from a per-expert stream so any
  one expert can be regenerated on its own;
* routing: each token picks k distinct experts by Gumbel-top-k over
  log-weights proportional to rank^-s (Zipf load); router probabilities are
  a softmax over k seeded N(0, 1) logits.

Seeds: activations 0, weights 1, routing 2, output gradients 3, probs 4.
"""
from __future__ import annotations

import numpy as np

SEED_ACT, SEED_W, SEED_ROUTE, SEED_DY, SEED_PROB = 0, 1, 2, 3, 4
BF16_MAX_BITS = 0x7F7F


def _rng(*seed) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(list(seed)))


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """float32 array -> bf16 bit patterns, round to nearest even (finite
    inputs).  Used to turn generated samples into bf16 tensors."""
    u = np.ascontiguousarray(a, np.float32).view(np.uint32)
    r = u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return (r >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, np.uint16).astype(np.uint32)
            << np.uint32(16)).view(np.float32)


def tiny_contract_tensor(rows: int = 128, cols: int = 256,
                         seed: int = SEED_ACT) -> np.ndarray:
    """N(0,1) with 1 % of entries x50 (outside the special rows); row 1 all
    zero, row 2 all +bf16 max.  Returns bf16 bits [rows, cols]."""
    g = _rng(seed, 1)
    x = g.standard_normal((rows, cols), dtype=np.float32)
    n_out = int(round(0.01 * rows * cols))
    special = {1, 2}
    cand = np.array([i for i in range(rows * cols) if i // cols not in special])
    pos = g.choice(cand, size=n_out, replace=False)
    x.reshape(-1)[pos] *= 50.0
    b = f32_to_bf16_bits(x)
    b[1, :] = 0
    b[2, :] = BF16_MAX_BITS
    return b


def activations(tokens: int, hidden: int, seed: int = SEED_ACT,
                outlier_frac: float = 1e-3, outlier_scale: float = 100.0,
                outlier_channels: int = 8) -> np.ndarray:
    """Log-normal per-token magnitude x N(0,1) entries, with outlier_frac of
    all entries x outlier_scale inside outlier_channels fixed channels.
    Returns bf16 bits [tokens, hidden]."""
    g = _rng(seed, 2)
    chans = np.sort(g.choice(hidden, size=outlier_channels, replace=False))
    mag = g.lognormal(0.0, 1.0, size=(tokens, 1)).astype(np.float32)
    x = g.standard_normal((tokens, hidden), dtype=np.float32) * mag
    n_out = int(round(outlier_frac * tokens * hidden))
    n_out = min(n_out, tokens * outlier_channels)
    cells = g.choice(tokens * outlier_channels, size=n_out, replace=False)
    rows, ci = cells // outlier_channels, cells % outlier_channels
    x[rows, chans[ci]] *= outlier_scale
    return f32_to_bf16_bits(x)


def expert_weight(expert: int, rows: int, cols: int, std: float,
                  seed: int = SEED_W) -> np.ndarray:
    """One expert's [rows, cols] N(0, std^2) weight as bf16 bits, from its
    own stream (seed, expert)."""
    g = _rng(seed, 3, expert)
    w = g.standard_normal((rows, cols), dtype=np.float32) * np.float32(std)
    return f32_to_bf16_bits(w)


def expert_weights(num: int, rows: int, cols: int, std: float,
                   seed: int = SEED_W, tag: int = 0) -> np.ndarray:
    """[num, rows, cols] stacked expert weights (bf16 bits).  tag separates
    the FC1 and FC2 streams."""
    out = np.empty((num, rows, cols), np.uint16)
    for e in range(num):
        out[e] = expert_weight(e + tag * 100003, rows, cols, std, seed)
    return out


def zipf_weights(num_experts: int, s: float) -> np.ndarray:
    r = np.arange(1, num_experts + 1, dtype=np.float64)
    w = r ** (-s)
    return w / w.sum()


def route_topk(tokens: int, num_experts: int, k: int, p: np.ndarray,
               seed: int = SEED_ROUTE) -> np.ndarray:
    """k distinct experts per token by Gumbel-top-k over log p (sampling
    without replacement proportional to p).  The rank -> expert mapping is a
    seeded permutation so heavy experts are spread over the id range.
    Returns int32 [tokens, k]."""
    g = _rng(seed, 4)
    perm = g.permutation(num_experts)
    logp = np.log(p)[perm]
    gum = g.gumbel(size=(tokens, num_experts))
    keys = logp[None, :] + gum
    top = np.argpartition(-keys, k - 1, axis=1)[:, :k]
    # order the k picks by key, highest first
    kv = np.take_along_axis(keys, top, axis=1)
    order = np.argsort(-kv, axis=1, kind="stable")
    return np.take_along_axis(top, order, axis=1).astype(np.int32)


def zipf_routing(tokens: int, num_experts: int, k: int, s: float = 1.1,
                 seed: int = SEED_ROUTE) -> np.ndarray:
    return route_topk(tokens, num_experts, k, zipf_weights(num_experts, s), seed)


def uniform_routing(tokens: int, num_experts: int, k: int, seed: int = SEED_ROUTE):
    """Every expert equally likely (the balanced-load reference case)."""
    p = np.full(num_experts, 1.0 / num_experts)
    return route_topk(tokens, num_experts, k, p, seed)


def uniform_plus_zipf_routing(tokens: int, num_experts: int, k: int,
                              s: float = 1.1, seed: int = SEED_ROUTE):
    """Half uniform, half Zipf(s) expert load."""
    p = 0.5 / num_experts + 0.5 * zipf_weights(num_experts, s)
    return route_topk(tokens, num_experts, k, p, seed)


def router_probs(tokens: int, k: int, seed: int = SEED_PROB) -> np.ndarray:
    """Softmax over k seeded N(0,1) logits per token, float32 [tokens, k]."""
    g = _rng(seed, 5)
    z = g.standard_normal((tokens, k))
    z = np.exp(z - z.max(axis=1, keepdims=True))
    return (z / z.sum(axis=1, keepdims=True)).astype(np.float32)


def output_grad(rows: int, cols: int, seed: int = SEED_DY) -> np.ndarray:
    """dY ~ N(0, 1) bf16 bits."""
    g = _rng(seed, 6)
    return f32_to_bf16_bits(g.standard_normal((rows, cols), dtype=np.float32))


def normal_bf16(shape, std: float = 1.0, seed: int = 0) -> np.ndarray:
    g = _rng(seed, 7)
    return f32_to_bf16_bits(g.standard_normal(shape, dtype=np.float32)
                            * np.float32(std))


def boundary_tensor(cols: int = 256, seed: int = 0) -> np.ndarray:
    """Rows that sit on the encodings' edges (the pages' "boundary", "zeros"
    and "maxes" test sets): bf16 max with mixed signs, bf16 subnormals, rows
    whose outer scale is an FP32 subnormal, powers of two times the E4M3 and
    E2M1 grid points and midpoints, each nudged by -1, 0, +1 bf16 ulp, and
    all-zero rows.  Returns bf16 bits [rows, cols] with rows a multiple of 32.
    """
    g = _rng(seed, 8)
    rows = []
    # zeros and +-max
    rows.append(np.zeros(cols, np.uint16))
    m = np.full(cols, BF16_MAX_BITS, np.uint16)
    m[g.random(cols) < 0.5] |= 0x8000
    rows.append(m)
    rows.append(np.full(cols, BF16_MAX_BITS | 0x8000, np.uint16))
    # subnormal bf16 rows (exponent field 0), and a row of tiny normals
    rows.append(g.integers(1, 0x80, size=cols).astype(np.uint16)
                | (g.integers(0, 2, size=cols).astype(np.uint16) << 15))
    rows.append(g.integers(0x0080, 0x0400, size=cols).astype(np.uint16))
    # grid points and midpoints of E4M3 (x 2^k) and E2M1, +-1 ulp
    e4 = []
    for c in range(127):
        ex, mt = (c >> 3) & 15, c & 7
        e4.append(mt * 2.0 ** -9 if ex == 0 else (1 + mt / 8) * 2.0 ** (ex - 7))
    e4 = np.array(e4)
    mids4 = (e4[:-1] + e4[1:]) / 2
    e2 = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6.0])
    mids2 = (e2[:-1] + e2[1:]) / 2
    vals = np.concatenate([e4, mids4, e2, mids2]).astype(np.float32)
    base = f32_to_bf16_bits(vals)
    for k in (-20, 0, 7, 30):
        scaled = f32_to_bf16_bits(vals * np.float32(2.0 ** k))
        for d in (-1, 0, 1):
            v = scaled.astype(np.int32) + d
            v = np.clip(v, 1, 0x7F7F).astype(np.uint16)
            sel = g.choice(v.size, size=cols, replace=True)
            row = v[sel]
            row[g.random(cols) < 0.3] |= 0x8000
            rows.append(row)
    del base
    # rows whose amax is exactly 2688 * 2^k (outer scale a power of two),
    # and rows scaled so that the outer scale is an FP32 subnormal
    for i, k in enumerate((0, 20, -60, -100, -118, -124)):
        row = bf16_bits_to_f32(normal_bf16((cols,), std=1.0, seed=seed + 50 + i))
        top = np.float32(2688.0 * 2.0 ** k) if k > -100 else np.float32(2.0 ** k)
        rowf = row / np.max(np.abs(row)) * top
        r = f32_to_bf16_bits(rowf)
        r[int(np.argmax(np.abs(row)))] = f32_to_bf16_bits(np.array([top]))[0]
        rows.append(r)
    # pad to a multiple of 32 rows with random N(0,1) rows
    while len(rows) % 32:
        rows.append(normal_bf16((cols,), std=1.0, seed=seed + 1000 + len(rows)))
    return np.stack(rows).astype(np.uint16)
