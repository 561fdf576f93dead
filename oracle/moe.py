"""FC1 + SwiGLU, FC2, finalize and the whole layer (float64).

Test infrastructure only.

The pipeline is the one of the operator documentation, section 1: router ->
permute by expert -> GEMM1 -> activation -> GEMM2 -> un-permute -> weighted
sum.  Each GEMM is written as section 13's reference computation: dequantize
the expert's weights, then multiply the activation rows by them (float64
matmul as a library step; every product of a bf16 activation and a
dequantized weight is exact in float64).

Readings (the pages leave these open):
  * FC1 output column 2j is the gate and 2j+1 the linear value (interleaved
    SwiGLU, operator documentation section 8; the adjacent gate/linear pair
    of PR 32122).  With the concatenated layout (swiglu_fusion=2, section 8)
    column j is the gate and column I+j the linear value; swiglu_fusion=0 is
    read as interleaved, as the section says the QMoE operator treats it.
  * SwiGLU(G, L) = G * sigmoid(alpha*G) * (L + beta) with G = min(gate,
    limit) and L = clamp(linear, -limit, limit) (section 8); the defaults
    alpha=1, beta=0, limit=+inf are the standard SiLU(gate)*linear.
  * The activation h between FC1 and FC2 is kept in the activation dtype,
    bfloat16, rounded to nearest even from the exact value (the pages keep
    intermediates in the activation dtype and accumulate bf16 in float32,
    section 12.1, "Accumulation policy").  The FC2 result per expanded row
    is kept unrounded.
  * The NVFP4 per-expert global scale multiplies the whole dot product
    (it is a common factor of every weight of the expert).
  * finalize: out[t] = sum_j w[t, j] * y[row of (t, j)], the weighted
    un-permute (section 1; PR 31156), rounded to bfloat16 only by the caller
    when comparing.
"""
from __future__ import annotations

import numpy as np

from . import codecs
from .dequant import expert_weights_f64, fc_n
from .route import expert_maps, route_topk, route_topk_router_weights


def swiglu(gate, lin, alpha: float = 1.0, beta: float = 0.0, limit: float = np.inf) -> np.ndarray:
    G = np.minimum(np.asarray(gate, np.float64), limit)
    L = np.clip(np.asarray(lin, np.float64), -limit, limit)
    with np.errstate(over="ignore"):
        return G / (1.0 + np.exp(-alpha * G)) * (L + beta)


def _rows_of(offsets, e):
    return int(offsets[e]), int(offsets[e + 1])


def fc1_swiglu(x_bits, k: int, w1, s1, g1, fmt: str, offsets, p2e, act=None, cols=None):
    """x bf16 bits [T][H]; w1 [E][H][I] packed FP4 with s1 [E][H/B][2I], or FP8 w1 [E][2I][H]
    with s1 None -> (h bf16 bits [R][I], u float64 [R][2I]).

    act: {"alpha", "beta", "limit", "fusion"} (fusion 2 = concatenated
    gate | linear halves, otherwise interleaved).
    cols: optional array of h columns j to compute (others left 0); the FC1
    columns of each pair (2j and 2j+1, or j and I+j) are evaluated for each.
    """
    act = act or {}
    concat = act.get("fusion", 1) == 2
    x64 = codecs.bf16_to_f64(x_bits)
    E = w1.shape[0]
    N = fc_n(w1, fmt)
    I = N // 2
    R = int(offsets[E])
    u = np.zeros((R, N), dtype=np.float64)
    if cols is None:
        fcols = None
    elif concat:
        fcols = np.concatenate([np.asarray(cols), I + np.asarray(cols)])
    else:
        fcols = np.stack([2 * np.asarray(cols), 2 * np.asarray(cols) + 1], 1).reshape(-1)
    for e in range(E):
        lo, hi = _rows_of(offsets, e)
        if lo == hi:
            continue
        wd = expert_weights_f64(w1[e], None if s1 is None else s1[e], None if g1 is None else g1[e], fmt, fcols)
        toks = [int(p2e[p]) // k for p in range(lo, hi)]
        ue = x64[toks] @ wd
        if fcols is None:
            u[lo:hi] = ue
        else:
            u[lo:hi, fcols] = ue
    gate, lin = (u[:, :I], u[:, I:]) if concat else (u[:, 0::2], u[:, 1::2])
    h = swiglu(gate, lin, act.get("alpha", 1.0), act.get("beta", 0.0), act.get("limit", np.inf))
    hb = codecs.bf16_from_f64(h)
    if cols is not None:
        mask = np.zeros(I, bool)
        mask[np.asarray(cols)] = True
        hb = np.where(mask[None, :], hb, 0).astype(np.uint16)
    return hb, u


def fc2(h_bits, w2, s2, g2, fmt: str, offsets, cols=None) -> np.ndarray:
    """h bf16 bits [R][I]; w2 [E][I][H/2] packed FP4 (or FP8 [E][H][I]) -> y float64 [R][H]
    (or [R][len(cols)])."""
    h64 = codecs.bf16_to_f64(h_bits)
    E = w2.shape[0]
    N = fc_n(w2, fmt) if cols is None else len(cols)
    R = int(offsets[E])
    y = np.zeros((R, N), dtype=np.float64)
    for e in range(E):
        lo, hi = _rows_of(offsets, e)
        if lo == hi:
            continue
        wd = expert_weights_f64(w2[e], None if s2 is None else s2[e], None if g2 is None else g2[e], fmt, cols)
        y[lo:hi] = h64[lo:hi] @ wd
    return y


def finalize(y, topk_w, e2p, T: int, k: int) -> np.ndarray:
    """y [R][H] (permuted rows), topk_w [T][k], e2p [T*k] -> out float64 [T][H]."""
    y = np.asarray(y, np.float64)
    w = np.asarray(topk_w, np.float64)
    out = np.zeros((T, y.shape[1]), dtype=np.float64)
    for t in range(T):
        for j in range(k):
            out[t] += w[t, j] * y[int(e2p[t * k + j])]
    return out


def layer(inp, act=None, router_weights=None) -> dict:
    """The whole expert path on synth.LayerInputs; returns every intermediate.
    router_weights [T][E]: DeepSeek-style mixing weights (route.route_topk_router_weights)."""
    c = inp.cfg
    if router_weights is None:
        idx, wts = route_topk(inp.logits, c.k)
    else:
        idx, wts = route_topk_router_weights(inp.logits, router_weights, c.k)
    offsets, p2e, e2p = expert_maps(idx, c.E)
    h, u = fc1_swiglu(inp.x, c.k, inp.w1, inp.s1, inp.g1, c.fmt, offsets, p2e, act)
    y = fc2(h, inp.w2, inp.s2, inp.g2, c.fmt, offsets)
    out = finalize(y, wts, e2p, c.T, c.k)
    return dict(idx=idx, w=wts, offsets=offsets, p2e=p2e, e2p=e2p, u=u, h=h, y=y, out=out)
