"""Which bf16 roundings of h may differ between the GPU and the oracle.

h is the SwiGLU of float32-accumulated FC1 outputs rounded to bfloat16; the
oracle rounds the exact value.  Where the exact value sits within the float32
error bound of a rounding midpoint, both neighbours are correct results, and
one such flip of a large h element can move the layer output by more than the
output tolerance.  Test infrastructure only.
"""
import numpy as np

from oracle import codecs, dequant, moe


U32 = 2.0 ** -24


def fc1_abs_sum(L, off, p2e):
    """sum_k |x[k]| * |W1[e][k][n]| (global scale included) for every routed row p and FC1 column n."""
    c = L.cfg
    x = np.abs(codecs.bf16_to_f64(L.x))
    A = np.zeros((int(off[c.E]), 2 * c.I))
    for e in range(c.E):
        lo, hi = int(off[e]), int(off[e + 1])
        if lo < hi:
            wd = np.abs(dequant.expert_weights_f64(L.w1[e], None if L.s1 is None else L.s1[e], None if L.g1 is None else L.g1[e], c.fmt))
            A[lo:hi] = x[np.asarray(p2e[lo:hi]) // c.k] @ wd
    return A


def bf16_order(bits):
    """bf16 bit patterns -> integers in value order (adjacent values differ by 1)."""
    b = np.asarray(bits, np.int64)
    mag = b & 0x7FFF
    return np.where(b & 0x8000, -mag, mag)


def h_error_bound(L, u_ref, oact, off, p2e):
    """(exact h, bound on |float32 h - exact h|, underflow floor) per element.

    |fl32(u) - u| <= gamma * sum|x w| for any summation order (gamma = 2 n 2^-24
    with n = K + 16 roundings, each at most one ulp), carried through SwiGLU by
    its derivative (times 2 for the curvature over that interval), plus a few
    ulps of float32 for the SwiGLU's own operations.  Below float32's normal
    range the GPU's SwiGLU underflows (exp overflows, the sigmoid becomes 0):
    there any |h| up to |G (L + beta)| 2^-126 + 2^-126 is a float32 result."""
    c = L.cfg
    act = oact or {}
    al, be, lim = act.get("alpha", 1.0), act.get("beta", 0.0), act.get("limit", np.inf)
    A = fc1_abs_sum(L, off, p2e)
    n = c.H + 16
    gam = 2 * n * U32 / (1 - 2 * n * U32)
    I = u_ref.shape[1] // 2
    concat = act.get("fusion", 1) == 2   # gate = column j, linear = column I + j
    gsel, lsel = (slice(0, I), slice(I, None)) if concat else (slice(0, None, 2), slice(1, None, 2))
    gate, lin = u_ref[:, gsel], u_ref[:, lsel]
    G = np.minimum(gate, lim)
    Lc = np.clip(lin, -lim, lim)
    with np.errstate(over="ignore"):
        sg = 1.0 / (1.0 + np.exp(-al * G))
    d_gate = np.where(gate < lim, (sg + al * G * sg * (1 - sg)) * (Lc + be), 0.0)
    d_lin = np.where(np.abs(lin) < lim, G * sg, 0.0)
    hf = moe.swiglu(gate, lin, al, be, lim)
    dh = 2 * (np.abs(d_gate) * gam * A[:, gsel] + np.abs(d_lin) * gam * A[:, lsel]) + 16 * U32 * np.abs(hf)
    floor = (np.abs(G * (Lc + be)) + 1.0) * 2.0 ** -126
    return hf, dh, floor


def h_roundings_differ_only_at_ties(L, g_h, h_ref, u_ref, oact, off, p2e):
    """Every element where the GPU's h differs from the oracle's must be a
    correct rounding of some float32 evaluation within the error bound: its
    bf16 value within dh (the float32 bound of h_error_bound) plus half a bf16
    ulp (the final rounding) of the exact value -- a rounding tie is the
    common case, several ulps occur only where dh itself spans them (a linear
    value that is a near-cancellation) -- or a float32 underflow (exact and
    GPU values both under the floor of h_error_bound).  Returns the number of
    differing elements."""
    diff = np.asarray(g_h) != np.asarray(h_ref)
    if not diff.any():
        return 0
    hf, dh, floor = h_error_bound(L, u_ref, oact, off, p2e)
    gv = codecs.bf16_to_f64(g_h)
    half_ulp = np.ldexp(1.0, np.frexp(np.where(gv == 0, 2.0 ** -133, gv))[1] - 9)   # half of bf16's 2^(e-8) spacing
    within = np.abs(gv - hf) <= dh + half_ulp
    under = (np.abs(hf) <= floor) & (np.abs(gv) <= floor)
    bad = diff & ~(within | under)
    assert not bad.any(), ("h differs beyond a rounding tie", np.argwhere(bad)[:8].tolist())
    return int(diff.sum())
