"""Pins of the oracles' MoE composition at E > 1, k > 1 (CPU only).

"MoE and QMoE -- CUDA Operator Documentation", sections 1 and 13, define the
layer per token: out[t] = sum_j w[t, j] * FFN_{e(t, j)}(x[t]), where e(t, j)
is the j-th selected expert of token t and FFN_e(x) = SwiGLU(x W1_e) W2_e,
with h rounded to the activation dtype (bf16) between the two GEMMs.  The
reference below computes exactly that, token by token, with no expert maps
at all: the selection comes from a lexicographic sort of (-logit, expert),
the weights from scipy's softmax (or the router_weights gather), the
weights from a per-nibble golden-table dequant, the products from torch
float64 matmuls.  Both oracles (numpy and C++) permute rows by expert,
gather x through perm_to_expanded and un-permute through expanded_to_perm;
a mix-up of any of those maps (p2e for e2p, token for expanded row, the
weight of the wrong slot) changes out or h here and fails.

The permuted h is compared bit for bit against an independent order: rows
sorted by (expert, expanded row t*k + j) with numpy's lexsort.
"""
import numpy as np
import pytest
import scipy.special
import torch

import synth
from oracle import codecs, cpp, moe
from test_oracle_math import table_dequant

# hot experts (every token picks the three) and ties across selection edges
CASES = [
    synth.shrink(synth.MTP8, E=16, T=6, k=4, H=64, I=32, seed=61),
    synth.shrink(synth.MX_DECODE, E=12, T=5, k=3, H=64, I=32, seed=62),
    synth.shrink(synth.DECODE, E=9, T=7, k=5, H=32, I=16, seed=63),
]


def _with_ties(L):
    """Copies an equal logit onto a second expert in every token (one inside
    the selected set, one at its edge), so the tie rule decides selections."""
    lg = L.logits.copy()
    for t in range(lg.shape[0]):
        order = np.lexsort((np.arange(lg.shape[1]), -lg[t].astype(np.float64)))
        k = L.cfg.k
        lg[t, order[k]] = lg[t, order[k - 1]]            # tie at the edge of the selected set
        lg[t, order[-1]] = lg[t, order[0]]               # tie at the top
    L.logits[:] = lg
    return L


def _swiglu_t(gate, lin, alpha, beta, limit):
    G = torch.clamp(gate, max=limit)
    Lc = torch.clamp(lin, min=-limit, max=limit)
    return G * torch.sigmoid(alpha * G) * (Lc + beta)


def direct_layer(L, act=None, rw=None):
    """Per-token definition: -> (out float64 [T][H], h bits in permuted order [T*k][I],
    offsets, p2e, e2p built by a lexsort over (expert, expanded row))."""
    c = L.cfg
    act = act or {}
    alpha, beta, limit = act.get("alpha", 1.0), act.get("beta", 0.0), act.get("limit", np.inf)
    concat = act.get("fusion", 1) == 2
    x = torch.tensor(codecs.bf16_to_f64(L.x))
    lg = L.logits.astype(np.float64)
    cache = {}

    def dense(e):
        if e not in cache:
            W1 = torch.tensor(table_dequant(L.w1[e], L.s1[e], None if L.g1 is None else L.g1[e], c.fmt))
            W2 = torch.tensor(table_dequant(L.w2[e], L.s2[e], None if L.g2 is None else L.g2[e], c.fmt))
            cache[e] = (W1, W2)
        return cache[e]

    out = np.zeros((c.T, c.H))
    rows = []                                   # (expert, expanded row, h bits)
    for t in range(c.T):
        sel = np.lexsort((np.arange(c.E), -lg[t]))[:c.k]
        w = (scipy.special.softmax(lg[t, sel]) if rw is None
             else rw[t, sel].astype(np.float64))
        for j, e in enumerate(sel):
            W1, W2 = dense(int(e))
            u = x[t] @ W1
            gate, lin = (u[:c.I], u[c.I:]) if concat else (u[0::2], u[1::2])
            hb = codecs.bf16_from_f64(_swiglu_t(gate, lin, alpha, beta, limit).numpy())
            v = torch.tensor(codecs.bf16_to_f64(hb)) @ W2
            out[t] += w[j] * v.numpy()
            rows.append((int(e), t * c.k + j, hb))
    e_arr = np.array([r[0] for r in rows])
    r_arr = np.array([r[1] for r in rows])
    order = np.lexsort((r_arr, e_arr))
    h_perm = np.stack([rows[i][2] for i in order])
    offsets = np.concatenate([[0], np.cumsum(np.bincount(e_arr, minlength=c.E))]).astype(np.int32)
    p2e = r_arr[order].astype(np.int32)
    e2p = np.empty_like(p2e)
    e2p[p2e] = np.arange(len(p2e), dtype=np.int32)
    return out, h_perm, offsets, p2e, e2p


def _compare(got, ref_out, ref_h, ref_off, ref_p2e, ref_e2p):
    np.testing.assert_array_equal(got["offsets"], ref_off)
    np.testing.assert_array_equal(got["p2e"], ref_p2e)
    np.testing.assert_array_equal(got["e2p"], ref_e2p)
    np.testing.assert_array_equal(got["h"], ref_h)
    scale = np.sqrt(np.mean(ref_out ** 2, axis=-1, keepdims=True))
    err = np.abs(got["out"] - ref_out)
    assert np.all(err <= 1e-12 * (np.abs(ref_out) + scale)), float(np.max(err / scale))


@pytest.mark.parametrize("oracle", ["numpy", "cpp"])
@pytest.mark.parametrize("variant", ["standard", "gptoss_concat", "router_weights"])
@pytest.mark.parametrize("cfg", CASES, ids=lambda c: c.name)
def test_layer_equals_per_token_definition(cfg, variant, oracle):
    L = _with_ties(synth.layer_inputs(cfg))
    act = dict(alpha=1.702, beta=1.0, limit=7.0, fusion=2) if variant == "gptoss_concat" else None
    rw = synth.router_weights(cfg) if variant == "router_weights" else None
    got = (moe if oracle == "numpy" else cpp).layer(L, act=act, router_weights=rw)
    _compare(got, *direct_layer(L, act, rw))


def test_composition_pin_rejects_planted_map_mistakes():
    """The pin fails when the oracle's un-permute takes p2e for e2p, or FC1
    gathers x by expanded row instead of token (mistakes planted in copies
    of the oracle's own steps, on the CPU)."""
    cfg = CASES[0]
    L = synth.layer_inputs(cfg)
    c = L.cfg
    ref = direct_layer(L)
    good = moe.layer(L)
    _compare(good, *ref)
    # finalize through the wrong map
    bad_out = moe.finalize(good["y"], good["w"], good["p2e"], c.T, c.k)
    with pytest.raises(AssertionError):
        _compare(dict(good, out=bad_out), *ref)
    # FC1 rows gathered by expanded row index instead of token (p2e taken for p2e // k)
    h_bad, _ = moe.fc1_swiglu(L.x, 1, L.w1, L.s1, L.g1, c.fmt, good["offsets"], good["p2e"] % c.T)
    with pytest.raises(AssertionError):
        _compare(dict(good, h=h_bad), *ref)
