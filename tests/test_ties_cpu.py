"""CPU checks of the h rounding-tie rule used by the end-to-end GPU parity checks.

A float32 emulation of FC1 (float32 matmul per expert, float32 global scale
and SwiGLU, bf16 round-to-nearest-even) stands in for the GPU: its h must be
accepted, and mistakes planted in it (a one-ulp change away from a tie, a
two-ulp change at a tie) must be rejected.
"""
import numpy as np
import pytest

import synth
from oracle import codecs, dequant, moe, route
from ties import bf16_order, h_error_bound, h_roundings_differ_only_at_ties

CFG = synth.shrink(synth.MTP8, E=32, T=8, k=8, H=512, I=256, seed=25)


def f32_fc1_h(L, off, p2e):
    c = L.cfg
    x = codecs.bf16_to_f64(L.x).astype(np.float32)
    u = np.zeros((int(off[c.E]), 2 * c.I), np.float32)
    for e in range(c.E):
        lo, hi = int(off[e]), int(off[e + 1])
        if lo < hi:
            wd = dequant.dequant_expert_f64(L.w1[e], L.s1[e], None, c.fmt).astype(np.float32)  # exact
            ue = x[np.asarray(p2e[lo:hi]) // c.k] @ wd
            u[lo:hi] = ue * np.float32(L.g1[e]) if L.g1 is not None else ue
    gate, lin = u[:, 0::2], u[:, 1::2]
    with np.errstate(over="ignore"):
        h = gate / (np.float32(1) + np.exp(-gate)) * lin
    return codecs.bf16_from_f32_bits(h.astype(np.float32))


@pytest.fixture(scope="module")
def case():
    L = synth.layer_inputs(CFG)
    idx, _ = route.route_topk(L.logits, CFG.k)
    off, p2e, _ = route.expert_maps(idx, CFG.E)
    h_ref, u_ref = moe.fc1_swiglu(L.x, CFG.k, L.w1, L.s1, L.g1, CFG.fmt, off, p2e)
    return L, off, p2e, h_ref, u_ref, f32_fc1_h(L, off, p2e)


def test_float32_emulation_is_accepted_and_has_ties(case):
    L, off, p2e, h_ref, u_ref, h32 = case
    ties = h_roundings_differ_only_at_ties(L, h32, h_ref, u_ref, None, off, p2e)
    assert ties > 0     # the case exercises the rule


def _step(bits, d):
    """bf16 bits moved d places in value order."""
    o = bf16_order(bits) + d
    return np.where(o < 0, 0x8000 | (-o), o).astype(np.uint16)


def test_one_ulp_away_from_a_tie_is_rejected(case):
    L, off, p2e, h_ref, u_ref, h32 = case
    hf, dh, floor = h_error_bound(L, u_ref, None, off, p2e)
    # the element farthest (in units of its bound) from a rounding midpoint
    ref = codecs.bf16_to_f64(h_ref)
    half_ulp = np.abs(codecs.bf16_to_f64(_step(h_ref, 1)) - ref) / 2
    margin = (half_ulp - np.abs(hf - ref)) / dh
    margin[np.abs(hf) <= floor] = -np.inf
    i = np.unravel_index(np.argmax(margin), margin.shape)
    assert margin[i] > 1.5
    bad = h_ref.copy()
    bad[i] = _step(bad[i], 1)
    with pytest.raises(AssertionError, match="rounding tie"):
        h_roundings_differ_only_at_ties(L, bad, h_ref, u_ref, None, off, p2e)


def test_large_value_set_to_zero_is_rejected(case):
    L, off, p2e, h_ref, u_ref, h32 = case
    i = np.unravel_index(np.argmax(np.abs(codecs.bf16_to_f64(h_ref))), h_ref.shape)
    bad = h32.copy()
    bad[i] = 0
    with pytest.raises(AssertionError, match="rounding tie"):
        h_roundings_differ_only_at_ties(L, bad, h_ref, u_ref, None, off, p2e)


def test_two_ulps_at_a_tie_is_rejected(case):
    L, off, p2e, h_ref, u_ref, h32 = case
    hf, dh, floor = h_error_bound(L, u_ref, None, off, p2e)
    # the differing (tie) element whose float32 bound is tightest against its
    # bf16 ulp: the exact value lies within dh of the midpoint, so a value two
    # ulps from the oracle's is >= 1.5 ulp - dh from it, outside the accepted
    # dh + ulp/2 whenever dh < ulp/2
    cand = np.argwhere((h32 != h_ref) & (np.abs(hf) > floor))
    ulp = np.ldexp(1.0, np.frexp(codecs.bf16_to_f64(h_ref))[1] - 8)
    i = tuple(min(cand, key=lambda c: dh[tuple(c)] / ulp[tuple(c)]))
    assert dh[i] < 0.4 * ulp[i]
    bad = h32.copy()
    bad[i] = _step(h_ref[i], 2 * int(np.sign(bf16_order(h32[i]) - bf16_order(h_ref[i]))))
    with pytest.raises(AssertionError, match="rounding tie"):
        h_roundings_differ_only_at_ties(L, bad, h_ref, u_ref, None, off, p2e)
