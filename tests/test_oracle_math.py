"""Pins for the oracle's routing, maps, dequant, FC1/FC2, finalize (CPU only).

Independent references: numpy's lexsort / stable argsort, scipy's softmax,
torch's fp8 and bfloat16 casts with the golden E2M1 table, brute-force loops
over the definition's indices on tiny shapes, closed forms (a single nonzero
code per column, powers of two), and the textbook dense SwiGLU FFN
(torch.nn.functional.silu) that an E=1, k=1 layer reduces to.
"""
import dataclasses

import numpy as np
import pytest
import scipy.special
import torch

import synth
from oracle import codecs, dequant, moe, route, tolerance
from test_oracle_codecs import golden_e2m1

E2M1 = golden_e2m1()


def torch_scale(byte, fmt):
    t = torch.from_numpy(np.ascontiguousarray(byte, np.uint8))
    dt = torch.float8_e4m3fn if fmt == "nvfp4" else torch.float8_e8m0fnu
    return t.view(dt).to(torch.float64).numpy()


def table_dequant(w_e, s_e, g_e, fmt):
    """Independent dequant: golden table lookup per nibble, torch scale decode, python indexing."""
    B = 16 if fmt == "nvfp4" else 32
    K, half = w_e.shape
    out = np.zeros((K, 2 * half))
    sc = torch_scale(s_e, fmt)
    for k in range(K):
        for j in range(half):
            byte = int(w_e[k, j])
            for nib, n in ((byte & 15, 2 * j), (byte >> 4, 2 * j + 1)):
                out[k, n] = E2M1[nib] * sc[k // B, n] * (1.0 if g_e is None else float(g_e))
    return out


# ----------------------------------------------------------------- routing --

def test_topk_equals_full_sort_and_weights_are_softmax():
    rng = np.random.default_rng(0)
    lg = rng.standard_normal((16, 256)).astype(np.float32)
    idx, w = route.route_topk(lg, 8)
    for t in range(16):
        order = np.lexsort((np.arange(256), -lg[t].astype(np.float64)))
        assert idx[t].tolist() == order[:8].tolist()
        sm = scipy.special.softmax(lg[t, order[:8]].astype(np.float64))
        np.testing.assert_allclose(w[t], sm, rtol=1e-14, atol=0)
        assert abs(w[t].sum() - 1.0) < 1e-15


def test_topk_equals_renormalised_full_softmax():
    rng = np.random.default_rng(1)
    lg = rng.standard_normal((4, 64)).astype(np.float32)
    idx, w = route.route_topk(lg, 6)
    for t in range(4):
        full = scipy.special.softmax(lg[t].astype(np.float64))
        sel = full[idx[t]]
        np.testing.assert_allclose(w[t], sel / sel.sum(), rtol=1e-13)


def test_k1_weight_is_exactly_one_and_kE_is_full_softmax():
    rng = np.random.default_rng(2)
    lg = rng.standard_normal((3, 8)).astype(np.float32)
    _, w1 = route.route_topk(lg, 1)
    assert np.all(w1 == 1.0)
    idx, w = route.route_topk(lg, 8)
    for t in range(3):
        assert sorted(idx[t].tolist()) == list(range(8))
        np.testing.assert_allclose(w[t], scipy.special.softmax(lg[t].astype(np.float64))[idx[t]], rtol=1e-14)


def test_ties_go_to_lower_index_and_signed_zeros_tie():
    lg = np.array([[1.0, 3.0, 3.0, -0.0, 0.0, 3.0, -1.0, 0.0]], np.float32)
    idx, w = route.route_topk(lg, 6)
    assert idx[0].tolist() == [1, 2, 5, 0, 3, 4]
    assert w[0, 0] == w[0, 1] == w[0, 2]
    lg2 = np.zeros((1, 16), np.float32)
    idx2, w2 = route.route_topk(lg2, 4)
    assert idx2[0].tolist() == [0, 1, 2, 3] and np.all(w2 == 0.25)


def test_neg_inf_sorts_last():
    lg = np.array([[-np.inf, -1e30, 0.0, -np.inf]], np.float32)
    idx, w = route.route_topk(lg, 3)
    assert idx[0].tolist() == [2, 1, 0]
    assert w[0, 2] == 0.0


# -------------------------------------------------------------------- maps --

@pytest.mark.parametrize("T,E,k,seed", [(1, 8, 2, 0), (4, 256, 8, 1), (8, 256, 8, 2), (512, 256, 8, 3), (3, 5, 5, 4)])
def test_maps_equal_stable_argsort(T, E, k, seed):
    rng = np.random.default_rng(seed)
    idx = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    off, p2e, e2p = route.expert_maps(idx, E)
    flat = idx.reshape(-1)
    order = np.argsort(flat, kind="stable")
    assert np.array_equal(p2e, order)
    assert np.array_equal(e2p[p2e], np.arange(T * k))
    assert np.array_equal(off, np.concatenate([[0], np.cumsum(np.bincount(flat, minlength=E))]))
    assert off[-1] == T * k and np.all(np.diff(off) >= 0)


# ----------------------------------------------------------------- dequant --

@pytest.mark.parametrize("fmt", ["nvfp4", "mxfp4"])
def test_dequant_f64_equals_table_bruteforce(fmt):
    cfg = synth.shrink(synth.TINY if fmt == "nvfp4" else synth.MX_DECODE, E=2, H=64, I=32, seed=11)
    L = synth.layer_inputs(cfg)
    for e in range(2):
        g = None if L.g1 is None else L.g1[e]
        np.testing.assert_array_equal(dequant.dequant_expert_f64(L.w1[e], L.s1[e], g, fmt),
                                      table_dequant(L.w1[e], L.s1[e], g, fmt))


@pytest.mark.parametrize("fmt", ["nvfp4", "mxfp4"])
def test_dequant_bf16_matches_torch_float32_path(fmt):
    cfg = synth.DequantConfig("t", fmt, E=3, K=128, N=96, seed=5)
    w, s, g = synth.dequant_inputs(cfg)
    got = dequant.dequant_bf16(w, s, g, fmt)
    B = cfg.B
    for e in range(3):
        codes = codecs.unpack_codes(w[e])
        val = torch.tensor(np.vectorize(E2M1.get)(codes), dtype=torch.float32)
        sc = torch.from_numpy(np.repeat(torch_scale(s[e], fmt), B, axis=0)).to(torch.float32)
        p = val * sc                                   # exact in float32
        if g is not None:
            p = p * torch.tensor(float(g[e]), dtype=torch.float32)   # one float32 RNE rounding
        ref = p.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).T
        np.testing.assert_array_equal(got[e], ref)


def test_mxfp4_dequant_is_exact_and_roundtrips():
    w, s, g = synth.dequant_inputs(synth.DequantConfig("t", "mxfp4", E=2, K=64, N=64, seed=9))
    out = codecs.bf16_to_f64(dequant.dequant_bf16(w, s, g, "mxfp4"))      # [E][N][K]
    for e in range(2):
        sc = np.repeat(torch_scale(s[e], "mxfp4"), 32, axis=0).T         # [N][K]
        back = out[e] / sc
        codes = codecs.unpack_codes(w[e]).T
        expect = np.vectorize(E2M1.get)(codes)
        np.testing.assert_array_equal(back, expect)


# ----------------------------------------------------------------- SwiGLU --

def test_swiglu_standard_equals_torch_silu_times_linear():
    rng = np.random.default_rng(4)
    g = rng.standard_normal(1000) * 10
    l = rng.standard_normal(1000) * 10
    ref = (torch.nn.functional.silu(torch.tensor(g)) * torch.tensor(l)).numpy()
    np.testing.assert_allclose(moe.swiglu(g, l), ref, rtol=1e-14, atol=1e-300)


def test_swiglu_special_cases():
    assert moe.swiglu(0.0, 5.0) == 0.0
    assert moe.swiglu(800.0, 3.0) == 2400.0
    v = moe.swiglu(-800.0, 3.0)
    assert v == 0.0 and np.signbit(v)
    # GPT-OSS variant clamps: G <= limit, -limit <= L <= limit
    a, b, lim = 1.702, 1.0, 7.0
    assert moe.swiglu(100.0, 100.0, a, b, lim) == pytest.approx(7.0 / (1 + np.exp(-a * 7.0)) * 8.0, rel=1e-15)
    assert moe.swiglu(1.0, -100.0, a, b, lim) == pytest.approx(1.0 / (1 + np.exp(-a)) * (-6.0), rel=1e-15)


# ------------------------------------------------------------ FC1 / FC2 ----

def _tiny_layer(fmt, seed=0, E=3, H=64, I=32, T=3, k=2):
    """fmt "mxfp4_g": MXFP4 with per-expert global scales."""
    base = synth.TINY if fmt == "nvfp4" else synth.MX_DECODE
    cfg = synth.shrink(base, E=E, H=H, I=I, T=T, k=k, seed=seed)
    if fmt == "mxfp4_g":
        cfg = dataclasses.replace(cfg, mx_global=True)
    return synth.layer_inputs(cfg)


def torch_fp8_weights(w_e, g_e):
    """Independent FP8 decode: torch's float8_e4m3fn cast of the [N][K] bytes, times g, as [K][N]."""
    v = torch.from_numpy(np.ascontiguousarray(w_e, np.uint8)).view(torch.float8_e4m3fn).to(torch.float64)
    return v.numpy().T * float(g_e)


@pytest.mark.parametrize("fmt_case", ["nvfp4", "mxfp4", "mxfp4_g", "fp8"])
def test_fc1_fc2_equal_bruteforce_loops(fmt_case):
    if fmt_case == "fp8":
        L = synth.layer_inputs(synth.shrink(synth.FP8_MTP4, E=3, H=64, I=32, T=3, k=2, seed=0))
        fmt = "fp8"
    else:
        L = _tiny_layer(fmt_case)
        fmt = "nvfp4" if fmt_case == "nvfp4" else "mxfp4"
    assert (L.g1 is None) == (fmt_case == "mxfp4")
    c = L.cfg
    idx, _ = route.route_topk(L.logits, c.k)
    off, p2e, _ = route.expert_maps(idx, c.E)
    h, u = moe.fc1_swiglu(L.x, c.k, L.w1, L.s1, L.g1, fmt, off, p2e)
    y = moe.fc2(h, L.w2, L.s2, L.g2, fmt, off)
    x64 = codecs.bf16_to_f64(L.x)
    h64 = codecs.bf16_to_f64(h)
    for e in range(c.E):
        if fmt == "fp8":
            W1, W2 = torch_fp8_weights(L.w1[e], L.g1[e]), torch_fp8_weights(L.w2[e], L.g2[e])
        else:
            W1 = table_dequant(L.w1[e], L.s1[e], None if L.g1 is None else L.g1[e], fmt)
            W2 = table_dequant(L.w2[e], L.s2[e], None if L.g2 is None else L.g2[e], fmt)
        for p in range(off[e], off[e + 1]):
            t = p2e[p] // c.k
            for n in range(2 * c.I):
                assert u[p, n] == pytest.approx(sum(x64[t, kk] * W1[kk, n] for kk in range(c.H)), rel=1e-12, abs=1e-9)
            for n in range(c.H):
                assert y[p, n] == pytest.approx(sum(h64[p, i] * W2[i, n] for i in range(c.I)), rel=1e-12, abs=1e-9)


def test_fc1_single_code_per_column_closed_form():
    # One nonzero code per column: u = x_k * e2m1 * scale * g exactly.
    K, N = 32, 8
    w = np.zeros((1, K, N // 2), np.uint8)
    s = np.full((1, K // 16, N), 0x38, np.uint8)          # E4M3 1.0
    s[0, 1, :] = 0x48                                     # E4M3 4.0 for k in 16..31
    rows = [3, 17, 5, 30, 0, 31, 16, 9]
    codes = [7, 15, 1, 9, 2, 5, 12, 6]
    for n, (kk, c) in enumerate(zip(rows, codes)):
        w[0, kk, n // 2] |= (c << (4 * (n % 2)))
    g = np.array([np.float32(1.25)])
    x = synth.to_bf16_bits(np.linspace(-2, 2, K, dtype=np.float32)[None, :])
    off = np.array([0, 1], np.int32)
    p2e = np.array([0], np.int32)
    _, u = moe.fc1_swiglu(x, 1, w, s, g, "nvfp4", off, p2e)
    x64 = codecs.bf16_to_f64(x)[0]
    for n, (kk, c) in enumerate(zip(rows, codes)):
        sc = 4.0 if kk >= 16 else 1.0
        assert u[0, n] == x64[kk] * E2M1[c] * sc * 1.25


def test_fc_linearity_power_of_two():
    L = _tiny_layer("nvfp4", seed=3)
    c = L.cfg
    idx, _ = route.route_topk(L.logits, c.k)
    off, p2e, _ = route.expert_maps(idx, c.E)
    _, u1 = moe.fc1_swiglu(L.x, c.k, L.w1, L.s1, L.g1, "nvfp4", off, p2e)
    x8 = (L.x.astype(np.uint32) + np.where((L.x & 0x7FFF) != 0, 3 << 7, 0)).astype(np.uint16)   # x * 8
    _, u8 = moe.fc1_swiglu(x8, c.k, L.w1, L.s1, L.g1, "nvfp4", off, p2e)
    np.testing.assert_array_equal(u8, 8.0 * u1)
    wz = np.zeros_like(L.w1)
    _, uz = moe.fc1_swiglu(L.x, c.k, wz, L.s1, L.g1, "nvfp4", off, p2e)
    assert np.all(uz == 0.0)


def test_layer_E1_k1_is_dense_swiglu_ffn():
    L = _tiny_layer("nvfp4", seed=6, E=1, T=5, k=1, H=64, I=48)
    r = moe.layer(L)
    W1 = torch.tensor(table_dequant(L.w1[0], L.s1[0], L.g1[0], "nvfp4"))
    W2 = torch.tensor(table_dequant(L.w2[0], L.s2[0], L.g2[0], "nvfp4"))
    x = torch.tensor(codecs.bf16_to_f64(L.x))
    u = x @ W1
    h = torch.nn.functional.silu(u[:, 0::2]) * u[:, 1::2]
    h = h.to(torch.float32).to(torch.bfloat16).to(torch.float64)   # bf16 intermediate
    ref = (h @ W2).numpy()
    assert np.all(r["w"] == 1.0)
    ok, rep = tolerance.check(r["out"], ref)
    # the float32 hop before bf16 can differ from one rounding by an ulp of h
    assert ok, rep
    np.testing.assert_allclose(r["u"], u.numpy(), rtol=1e-13)


def _concat_to_interleaved(w, s):
    """Column permutation written out nibble by nibble: interleaved column 2j
    takes concatenated column j (gate), 2j+1 takes column I+j (linear)."""
    E, K, half = w.shape
    I = half
    codes = np.zeros((E, K, 2 * half), np.uint8)
    for n in range(2 * half):
        codes[:, :, n] = (w[:, :, n // 2] >> (4 * (n % 2))) & 15
    perm = np.empty(2 * I, np.int64)
    perm[0::2] = np.arange(I)
    perm[1::2] = I + np.arange(I)
    ci = codes[:, :, perm]
    wi = (ci[:, :, 0::2] | (ci[:, :, 1::2] << 4)).astype(np.uint8)
    return wi, s[:, :, perm]


@pytest.mark.parametrize("fmt", ["nvfp4", "mxfp4"])
def test_concat_swiglu_equals_interleaved_on_permuted_columns(fmt):
    L = _tiny_layer(fmt, seed=11, E=4, T=4, k=2, H=64, I=32)
    c = L.cfg
    idx, _ = route.route_topk(L.logits, c.k)
    off, p2e, _ = route.expert_maps(idx, c.E)
    act = dict(alpha=1.702, beta=1.0, limit=7.0)
    hc, uc = moe.fc1_swiglu(L.x, c.k, L.w1, L.s1, L.g1, fmt, off, p2e, dict(act, fusion=2))
    wi, si = _concat_to_interleaved(L.w1, L.s1)
    hi, ui = moe.fc1_swiglu(L.x, c.k, wi, si, L.g1, fmt, off, p2e, dict(act, fusion=1))
    np.testing.assert_array_equal(hc, hi)
    np.testing.assert_array_equal(uc[:, :c.I], ui[:, 0::2])
    np.testing.assert_array_equal(uc[:, c.I:], ui[:, 1::2])
    # fusion 0 is read as interleaved
    h0, _ = moe.fc1_swiglu(L.x, c.k, wi, si, L.g1, fmt, off, p2e, dict(act, fusion=0))
    np.testing.assert_array_equal(h0, hi)
    # sampled columns give the same values as the full computation
    cols = np.array([0, 5, 31])
    hs, _ = moe.fc1_swiglu(L.x, c.k, L.w1, L.s1, L.g1, fmt, off, p2e, dict(act, fusion=2), cols=cols)
    np.testing.assert_array_equal(hs[:, cols], hc[:, cols])


def test_concat_layer_E1_k1_is_dense_swiglu_ffn():
    L = _tiny_layer("nvfp4", seed=12, E=1, T=4, k=1, H=64, I=48)
    r = moe.layer(L, act=dict(fusion=2))
    W1 = torch.tensor(table_dequant(L.w1[0], L.s1[0], L.g1[0], "nvfp4"))
    x = torch.tensor(codecs.bf16_to_f64(L.x))
    u = x @ W1
    h = torch.nn.functional.silu(u[:, :48]) * u[:, 48:]
    hb = torch.tensor(codecs.bf16_to_f64(r["h"]))
    torch.testing.assert_close(hb, h, rtol=2 ** -8, atol=1e-30)


def test_router_weights_are_gathered_at_the_selection():
    rng = np.random.default_rng(13)
    T, E, k = 5, 40, 6
    lg = rng.standard_normal((T, E)).astype(np.float32)
    rw = (np.arange(T)[:, None] * 1000 + np.arange(E)[None, :] + 0.5).astype(np.float32)
    idx, w = route.route_topk_router_weights(lg, rw, k)
    ref_idx, _ = route.route_topk(lg, k)
    np.testing.assert_array_equal(idx, ref_idx)
    for t in range(T):
        order = np.lexsort((np.arange(E), -lg[t].astype(np.float64)))[:k]
        np.testing.assert_array_equal(idx[t], order)
        np.testing.assert_array_equal(w[t], t * 1000 + order + 0.5)   # row t, the chosen columns
    L = _tiny_layer("nvfp4", seed=14, E=6, T=3, k=2)
    rws = synth.router_weights(L.cfg)
    a = moe.layer(L, router_weights=rws)
    b = moe.layer(L)
    np.testing.assert_array_equal(a["idx"], b["idx"])
    np.testing.assert_array_equal(a["y"], b["y"])
    np.testing.assert_allclose(a["out"], moe.finalize(b["y"], rws[np.arange(3)[:, None], b["idx"]], b["e2p"], 3, 2),
                               rtol=1e-15)


def test_fp8_dequant_every_byte_matches_torch():
    # every byte value at every (n, k) position pattern; [E][N][K] layout
    E, N, K = 2, 16, 32
    w = (np.arange(E * N * K) * 37 % 256).astype(np.uint8).reshape(E, N, K)
    assert set(np.unique(w)) == set(range(256))
    g = np.array([1.0, 0.8125], np.float32)
    for e in range(E):
        got = dequant.dequant_fp8_expert_f64(w[e], g[e])
        ref = torch_fp8_weights(w[e], g[e])
        nan = np.isnan(ref)
        assert np.array_equal(np.isnan(got), nan) and nan.sum() == 2 * (N * K // 256)   # 0x7F, 0xFF
        np.testing.assert_array_equal(got[~nan], ref[~nan])
        cols = np.array([3, 0, 15])
        np.testing.assert_array_equal(dequant.dequant_fp8_expert_f64(w[e], g[e], cols)[:, :2],
                                      got[:, cols[:2]])
    # bf16 output: torch's float32 product, then its bfloat16 cast
    gb = np.array([1.3, 0.6], np.float32)
    wb = np.where((w & 0x7F) == 0x7F, 0, w).astype(np.uint8)          # finite bytes only
    got = dequant.dequant_fp8_bf16(wb, gb)
    for e in range(E):
        t = torch.from_numpy(wb[e]).view(torch.float8_e4m3fn).to(torch.float32) * float(gb[e])
        ref = t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        np.testing.assert_array_equal(got[e], ref)


def test_fp8_layer_E1_k1_is_dense_swiglu_ffn():
    L = synth.layer_inputs(synth.shrink(synth.FP8_MTP4, E=1, T=5, k=1, H=64, I=48, seed=15))
    r = moe.layer(L)
    W1 = torch.tensor(torch_fp8_weights(L.w1[0], L.g1[0]))
    W2 = torch.tensor(torch_fp8_weights(L.w2[0], L.g2[0]))
    x = torch.tensor(codecs.bf16_to_f64(L.x))
    u = x @ W1
    h = torch.nn.functional.silu(u[:, 0::2]) * u[:, 1::2]
    np.testing.assert_allclose(r["u"], u.numpy(), rtol=1e-13)
    hb = torch.tensor(codecs.bf16_to_f64(r["h"]))
    torch.testing.assert_close(hb, h, rtol=2 ** -8, atol=1e-30)
    ref = (hb @ W2).numpy()
    np.testing.assert_allclose(r["y"], ref, rtol=1e-12)


def test_finalize_k1_and_identical_rows():
    rng = np.random.default_rng(8)
    y = rng.standard_normal((6, 10))
    out = moe.finalize(y, np.ones((6, 1)), np.arange(6), 6, 1)
    np.testing.assert_array_equal(out, y)
    yk = np.repeat(rng.standard_normal((1, 10)), 4, axis=0)
    w = scipy.special.softmax(rng.standard_normal(4))[None, :]
    out = moe.finalize(yk, w, np.array([2, 0, 3, 1]), 1, 4)
    np.testing.assert_allclose(out[0], yk[0], rtol=1e-15)


def test_tolerance_rule():
    ok, _ = tolerance.check([1.0, 2.0], [1.0 + 1e-3, 2.0])
    assert ok
    ok, rep = tolerance.check([1.2], [1.0])
    assert not ok and rep["n_bad"] == 1
    ok, _ = tolerance.check([np.nan], [1.0])
    assert not ok
