"""Softmax top-k routing and the expert maps (float64 / integers).

Test infrastructure only.

Routing (operator documentation section 1: "router (top-k softmax) ->
permute by expert"; PR 31156: selection with a stable packed key, ties
unchanged across kernels).  Readings:
  * the k experts are chosen on the raw float32 logits, largest first, ties
    to the lower expert index, -0 equal to +0;
  * the k weights are a softmax over the selected logits (equivalently the
    softmax over all E experts renormalised over the k chosen), so they sum
    to 1;
  * with router_weights (operator documentation section 2, input 14,
    DeepSeek-style routing) the logits only choose the experts and the k
    mixing weights are router_weights[t, e] at the chosen experts, taken as
    they are (no softmax, no renormalisation).

Expert maps (PR 31156, the expert-map prologue; operator documentation
section 1, "permute by expert"): expanded row r = t*k + j; rows are grouped
by expert in ascending expert order, and inside an expert by ascending r
(a stable counting sort).
"""
from __future__ import annotations

import math

import numpy as np


def route_topk(logits, k: int):
    """logits float32 [T][E] -> (idx int32 [T][k], weights float64 [T][k])."""
    lg = np.asarray(logits, dtype=np.float32)
    T, E = lg.shape
    idx = np.zeros((T, k), dtype=np.int32)
    wts = np.zeros((T, k), dtype=np.float64)
    for t in range(T):
        row = [float(v) for v in lg[t]]
        order = sorted(range(E), key=lambda e: (-row[e], e))   # -0.0 == 0.0 in Python
        sel = order[:k]
        lmax = row[sel[0]]
        ex = [math.exp(row[e] - lmax) for e in sel]
        tot = math.fsum(ex)
        idx[t] = sel
        wts[t] = [v / tot for v in ex]
    return idx, wts


def expert_maps(idx, E: int):
    """idx [T][k] -> (offsets [E+1], perm_to_expanded [T*k], expanded_to_perm [T*k])."""
    flat = [int(v) for v in np.asarray(idx).reshape(-1)]
    R = len(flat)
    count = [0] * E
    for e in flat:
        count[e] += 1
    offsets = [0] * (E + 1)
    for e in range(E):
        offsets[e + 1] = offsets[e] + count[e]
    seen = [0] * E
    p2e = [0] * R
    e2p = [0] * R
    for r, e in enumerate(flat):
        p = offsets[e] + seen[e]
        seen[e] += 1
        p2e[p] = r
        e2p[r] = p
    return (np.array(offsets, dtype=np.int32), np.array(p2e, dtype=np.int32),
            np.array(e2p, dtype=np.int32))


def route_topk_router_weights(logits, router_weights, k: int):
    """Selection on the logits as route_topk; mixing weights gathered from
    router_weights [T][E] at the selected experts (section 2, input 14)."""
    idx, _ = route_topk(logits, k)
    rw = np.asarray(router_weights, dtype=np.float32)
    wts = np.zeros(idx.shape, dtype=np.float64)
    for t in range(idx.shape[0]):
        for j in range(idx.shape[1]):
            wts[t, j] = float(rw[t, idx[t, j]])
    return idx, wts
