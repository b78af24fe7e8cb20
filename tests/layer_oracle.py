"""The MoE expert-layer forward computed by the CPU oracle alone, from the
raw bf16 inputs (routing, quantization, binary64 GEMMs, SwiGLU x prob,
combine).  Intermediate tensors are rounded to bf16 where the layer stores
bf16 (gate_up output, SwiGLU output, down output, layer output).

Token sampling: `tokens` restricts the computation to the rows those tokens
feed (their routed assignments and, with a shared expert, their shared
rows), which is exact because every stage is row-local."""
from __future__ import annotations

import numpy as np

import oracle


def _rows_for_tokens(off, src, T, k, tokens, shared):
    tok_of = oracle.route_token(src, T, k)
    rows = np.nonzero(np.isin(tok_of, tokens))[0]
    return rows


def _group_of(off, rows):
    return np.searchsorted(off, rows, side="right") - 1


def mxfp8_layer(x, ids, prob_flat, w1, w2, E, inter, tokens=None):
    """x [T, H], w1 [E, 2I, H], w2 [E, H, I] bf16 bits.  Returns dict."""
    T, H = x.shape
    k = ids.shape[1]
    off, src, slot = oracle.route(ids, E)
    tok = oracle.route_token(src, T, k)
    rows = np.arange(T * k) if tokens is None else _rows_for_tokens(off, src, T, k, tokens, False)
    grp = _group_of(off, rows)
    qx, sx = oracle.quantize_mxfp8_rowwise(x)
    A = oracle.decode_mxfp8(qx[tok[rows]], sx[tok[rows]])
    c = np.empty((rows.size, 2 * inter))
    wq = {}
    for e in np.unique(grp):
        q1, s1 = oracle.quantize_mxfp8_rowwise(w1[e])
        q2, s2 = oracle.quantize_mxfp8_rowwise(w2[e])
        wq[e] = (oracle.decode_mxfp8(q1, s1), oracle.decode_mxfp8(q2, s2))
        sel = grp == e
        c[sel] = A[sel] @ wq[e][0].T
    c16 = oracle.f64_to_bf16(c)
    d16 = oracle.f64_to_bf16(oracle.swiglu_prob(oracle.bf16_to_f64(c16), prob_flat[src[rows]]))
    qd, sd = oracle.quantize_mxfp8_rowwise(d16)
    D = oracle.decode_mxfp8(qd, sd)
    y = np.empty((rows.size, H))
    for e in np.unique(grp):
        sel = grp == e
        y[sel] = D[sel] @ wq[e][1].T
    y16 = oracle.f64_to_bf16(y)
    out = None
    if tokens is not None:
        pos = {int(r): i for i, r in enumerate(rows)}
        yv = oracle.bf16_to_f64(y16)
        out = np.stack([sum(yv[pos[int(slot[t, j])]] for j in range(k)) for t in tokens])
    else:
        out = oracle.combine(oracle.bf16_to_f64(y16), slot)
    return dict(off=off, src=src, tok=tok, slot=slot, rows=rows, qa=qx[tok[rows]],
                sa=sx[tok[rows]], c=c16, d=d16, qd=qd, sd=sd, y=y16,
                out=oracle.f64_to_bf16(out))


def nvfp4_layer(x, ids, prob_flat, w1, w2, E, inter, tokens=None, w1_of=None, w2_of=None):
    """Routed experts + shared expert (group E), per-token NVFP4
    activations, NVFP4 weights with one outer scale per expert tensor.
    w1 [E+1, 2I, H], w2 [E+1, H, I] bf16 bits, or None with w1_of(e) /
    w2_of(e) returning one expert's weights."""
    T, H = x.shape
    k = ids.shape[1]
    off, src, slot = oracle.route(ids, E, shared_expert=True)
    tok = oracle.route_token(src, T, k)
    rows = np.arange(T * k + T) if tokens is None else _rows_for_tokens(off, src, T, k, tokens, True)
    grp = _group_of(off, rows)
    prob_all = np.concatenate([np.asarray(prob_flat, np.float64), np.ones(T)])
    qx, sbx, sgx = oracle.quantize_nvfp4(x)
    A = oracle.decode_nvfp4(qx[tok[rows]], sbx[tok[rows]], sgx[tok[rows]])
    get1 = (lambda e: w1[e]) if w1 is not None else w1_of
    get2 = (lambda e: w2[e]) if w2 is not None else w2_of
    c = np.empty((rows.size, 2 * inter))
    wq = {}
    for e in np.unique(grp):
        a1, b1, g1 = oracle.quantize_nvfp4(get1(e), rows_per_group=2 * inter)
        a2, b2, g2 = oracle.quantize_nvfp4(get2(e), rows_per_group=H)
        wq[e] = (oracle.decode_nvfp4(a1, b1, g1, 2 * inter), oracle.decode_nvfp4(a2, b2, g2, H))
        sel = grp == e
        c[sel] = A[sel] @ wq[e][0].T
    c16 = oracle.f64_to_bf16(c)
    d16 = oracle.f64_to_bf16(oracle.swiglu_prob(oracle.bf16_to_f64(c16), prob_all[src[rows]]))
    qd, sbd, sgd = oracle.quantize_nvfp4(d16)
    D = oracle.decode_nvfp4(qd, sbd, sgd)
    y = np.empty((rows.size, H))
    for e in np.unique(grp):
        sel = grp == e
        y[sel] = D[sel] @ wq[e][1].T
    y16 = oracle.f64_to_bf16(y)
    yv = oracle.bf16_to_f64(y16)
    pos = {int(r): i for i, r in enumerate(rows)}
    toks = np.arange(T) if tokens is None else np.asarray(tokens)
    out = np.stack([sum(yv[pos[int(slot[t, j])]] for j in range(k)) + yv[pos[T * k + int(t)]]
                    for t in toks])
    return dict(off=off, src=src, tok=tok, slot=slot, rows=rows, qa=qx[tok[rows]],
                sba=sbx[tok[rows]], sga=sgx[tok[rows]], c=c16, d=d16, qd=qd, sbd=sbd,
                sgd=sgd, y=y16, out=oracle.f64_to_bf16(out))
