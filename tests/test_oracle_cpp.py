"""Pins for the C++ oracle (oracle/qmoe_oracle.cpp), CPU only.

The C++ oracle is pinned the same way as the numpy oracle -- against the
golden E2M1 table, torch's float8 and bfloat16 casts, a brute-force nearest-
bfloat16 search with exact rationals, numpy's lexsort / stable argsort,
scipy's softmax, brute-force loops over the definition's indices, closed
forms and the dense SwiGLU FFN an E=1, k=1 layer reduces to -- and, since the
two oracles were written independently and share no code, against the numpy
oracle on whole layers (bit-exact on every integer and bf16 output, 1e-12
relative on the float64 ones).
"""
import dataclasses

import numpy as np
import pytest
import scipy.special
import torch

import synth
from oracle import codecs, cpp, moe, route
from test_oracle_codecs import _nearest_bf16_bruteforce, golden_e2m1
from test_oracle_math import _concat_to_interleaved, _tiny_layer, table_dequant, torch_fp8_weights, torch_scale

E2M1 = golden_e2m1()


@pytest.fixture(scope="module", autouse=True)
def _lib():
    cpp.lib()        # compiles the oracle with g++ if the shared object is missing or stale


# ------------------------------------------------------------------ codecs --

def test_e2m1_all_codes_match_golden_table():
    got = cpp.e2m1_value(np.arange(16))
    for c in range(16):
        assert got[c] == E2M1[c] and np.signbit(got[c]) == np.signbit(E2M1[c]), c


def test_e4m3fn_and_e8m0_all_256_bytes_match_torch():
    b = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    for dt, fn, nan_count in ((torch.float8_e4m3fn, cpp.e4m3fn_value, 2), (torch.float8_e8m0fnu, cpp.e8m0_value, 1)):
        ref = b.view(dt).to(torch.float64).numpy()
        got = fn(np.arange(256))
        nan = np.isnan(ref)
        assert np.array_equal(np.isnan(got), nan) and nan.sum() == nan_count
        assert np.array_equal(got[~nan], ref[~nan])
        assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))
    assert cpp.e4m3fn_value([0x7E])[0] == 448.0 and cpp.e4m3fn_value([0x01])[0] == 2.0 ** -9


def test_bf16_from_f32_matches_torch():
    rng = np.random.default_rng(17)
    a = np.concatenate([
        rng.standard_normal(20000).astype(np.float32) * np.float32(1e3),
        rng.integers(0, 2 ** 32, 20000, dtype=np.uint64).astype(np.uint32).view(np.float32),
        np.array([0.0, -0.0, np.inf, -np.inf, 3.3895314e38, 1e-45, -1e-40], np.float32),
    ])
    ref = torch.from_numpy(a).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = cpp.bf16_from_f32_bits(a)
    nan = np.isnan(a)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.all((got[nan] & 0x7FC0) == 0x7FC0)


def test_bf16_from_f64_single_rounding_bruteforce():
    rng = np.random.default_rng(23)
    xs = list(rng.standard_normal(300) * 10.0 ** rng.integers(-40, 39, 300))
    xs += [1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, 1.0 + 2.0 ** -8 + 2.0 ** -40, 1.0 + 2.0 ** -8 - 2.0 ** -40,
           -(1.0 + 2.0 ** -8 + 2.0 ** -40), 2.0 ** -130 * 1.5, 2.0 ** -133 * 0.5, 2.0 ** -133 * 0.75,
           3.3961e38, 3.40e38, 0.0, -0.0]
    got = cpp.bf16_from_f64(np.array(xs))
    for x, gbits in zip(xs, got):
        assert int(gbits) == _nearest_bf16_bruteforce(float(x)), x


# ----------------------------------------------------------------- routing --

def test_topk_equals_full_sort_and_weights_are_softmax():
    rng = np.random.default_rng(30)
    lg = rng.standard_normal((16, 256)).astype(np.float32)
    idx, w = cpp.route_topk(lg, 8)
    for t in range(16):
        order = np.lexsort((np.arange(256), -lg[t].astype(np.float64)))
        assert idx[t].tolist() == order[:8].tolist()
        np.testing.assert_allclose(w[t], scipy.special.softmax(lg[t, order[:8]].astype(np.float64)), rtol=1e-14)
        full = scipy.special.softmax(lg[t].astype(np.float64))[order[:8]]
        np.testing.assert_allclose(w[t], full / full.sum(), rtol=1e-13)
        assert abs(w[t].sum() - 1.0) < 1e-15


def test_topk_ties_signed_zero_neg_inf_and_k_extremes():
    lg = np.array([[1.0, 3.0, 3.0, -0.0, 0.0, 3.0, -1.0, 0.0]], np.float32)
    idx, w = cpp.route_topk(lg, 6)
    assert idx[0].tolist() == [1, 2, 5, 0, 3, 4] and w[0, 0] == w[0, 1] == w[0, 2]
    idx, w = cpp.route_topk(np.array([[-np.inf, -1e30, 0.0, -np.inf]], np.float32), 3)
    assert idx[0].tolist() == [2, 1, 0] and w[0, 2] == 0.0
    rng = np.random.default_rng(31)
    lg = rng.standard_normal((3, 8)).astype(np.float32)
    _, w1 = cpp.route_topk(lg, 1)
    assert np.all(w1 == 1.0)
    idx, w = cpp.route_topk(lg, 8)
    for t in range(3):
        assert sorted(idx[t].tolist()) == list(range(8))
        np.testing.assert_allclose(w[t], scipy.special.softmax(lg[t].astype(np.float64))[idx[t]], rtol=1e-14)


def test_router_weights_are_gathered_at_the_selection():
    rng = np.random.default_rng(32)
    T, E, k = 5, 40, 6
    lg = rng.standard_normal((T, E)).astype(np.float32)
    rw = (np.arange(T)[:, None] * 1000 + np.arange(E)[None, :] + 0.5).astype(np.float32)
    idx, w = cpp.route_topk_router_weights(lg, rw, k)
    for t in range(T):
        order = np.lexsort((np.arange(E), -lg[t].astype(np.float64)))[:k]
        np.testing.assert_array_equal(idx[t], order)
        np.testing.assert_array_equal(w[t], t * 1000 + order + 0.5)


@pytest.mark.parametrize("T,E,k,seed", [(1, 8, 2, 0), (4, 256, 8, 1), (512, 256, 8, 3), (3, 5, 5, 4)])
def test_maps_equal_stable_argsort(T, E, k, seed):
    rng = np.random.default_rng(seed)
    idx = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    off, p2e, e2p = cpp.expert_maps(idx, E)
    flat = idx.reshape(-1)
    assert np.array_equal(p2e, np.argsort(flat, kind="stable"))
    assert np.array_equal(e2p[p2e], np.arange(T * k))
    assert np.array_equal(off, np.concatenate([[0], np.cumsum(np.bincount(flat, minlength=E))]))


# ----------------------------------------------------------------- dequant --

@pytest.mark.parametrize("fmt", ["nvfp4", "mxfp4"])
def test_dequant_matches_table_and_torch_float32_path(fmt):
    cfg = synth.DequantConfig("t", fmt, E=3, K=128, N=96, seed=5)
    w, s, g = synth.dequant_inputs(cfg)
    got = cpp.dequant_bf16(w, s, g, fmt)
    for e in range(3):
        ge = None if g is None else g[e]
        np.testing.assert_array_equal(cpp.expert_weights_f64(w, s, g, fmt, e), table_dequant(w[e], s[e], ge, fmt))
        codes = np.stack([w[e] & 15, w[e] >> 4], -1).reshape(cfg.K, cfg.N)
        val = torch.tensor(np.vectorize(E2M1.get)(codes), dtype=torch.float32)
        sc = torch.from_numpy(np.repeat(torch_scale(s[e], fmt), cfg.B, axis=0)).to(torch.float32)
        p = val * sc
        if ge is not None:
            p = p * torch.tensor(float(ge), dtype=torch.float32)
        ref = p.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).T
        np.testing.assert_array_equal(got[e], ref)


def test_fp8_dequant_every_byte_matches_torch():
    E, N, K = 2, 16, 32
    w = (np.arange(E * N * K) * 37 % 256).astype(np.uint8).reshape(E, N, K)
    g = np.array([1.0, 0.8125], np.float32)
    for e in range(E):
        got = cpp.expert_weights_f64(w, None, g, "fp8", e)
        ref = torch_fp8_weights(w[e], g[e])
        nan = np.isnan(ref)
        assert np.array_equal(np.isnan(got), nan)
        np.testing.assert_array_equal(got[~nan], ref[~nan])
    wb = np.where((w & 0x7F) == 0x7F, 0, w).astype(np.uint8)
    gb = np.array([1.3, 0.6], np.float32)
    got = cpp.dequant_bf16(wb, None, gb, "fp8")
    for e in range(E):
        t = torch.from_numpy(wb[e]).view(torch.float8_e4m3fn).to(torch.float32) * float(gb[e])
        np.testing.assert_array_equal(got[e], t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16))


# ------------------------------------------------------------ FC1 / FC2 ----

@pytest.mark.parametrize("fmt_case", ["nvfp4", "mxfp4", "mxfp4_g", "fp8"])
def test_fc1_fc2_equal_bruteforce_loops(fmt_case):
    if fmt_case == "fp8":
        L = synth.layer_inputs(synth.shrink(synth.FP8_MTP4, E=3, H=64, I=32, T=3, k=2, seed=0))
        fmt = "fp8"
    else:
        L = _tiny_layer(fmt_case)
        fmt = "nvfp4" if fmt_case == "nvfp4" else "mxfp4"
    c = L.cfg
    idx, _ = cpp.route_topk(L.logits, c.k)
    off, p2e, _ = cpp.expert_maps(idx, c.E)
    h, u = cpp.fc1_swiglu(L.x, c.k, L.w1, L.s1, L.g1, fmt, off, p2e)
    y = cpp.fc2(h, L.w2, L.s2, L.g2, fmt, off)
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
            g_, l_ = u[p, 0::2], u[p, 1::2]
            silu = torch.nn.functional.silu(torch.tensor(g_)).numpy() * l_
            np.testing.assert_allclose(codecs.bf16_to_f64(h[p]), silu, rtol=2 ** -8, atol=1e-30)
            for n in range(c.H):
                assert y[p, n] == pytest.approx(sum(h64[p, i] * W2[i, n] for i in range(c.I)), rel=1e-12, abs=1e-9)


def test_fc1_single_code_per_column_closed_form():
    K, N = 32, 8
    w = np.zeros((1, K, N // 2), np.uint8)
    s = np.full((1, K // 16, N), 0x38, np.uint8)          # E4M3 1.0
    s[0, 1, :] = 0x48                                     # E4M3 4.0 for k in 16..31
    rows = [3, 17, 5, 30, 0, 31, 16, 9]
    codes = [7, 15, 1, 9, 2, 5, 12, 6]
    for n, (kk, cc) in enumerate(zip(rows, codes)):
        w[0, kk, n // 2] |= (cc << (4 * (n % 2)))
    g = np.array([np.float32(1.25)])
    x = synth.to_bf16_bits(np.linspace(-2, 2, K, dtype=np.float32)[None, :])
    _, u = cpp.fc1_swiglu(x, 1, w, s, g, "nvfp4", np.array([0, 1], np.int32), np.array([0], np.int32))
    x64 = codecs.bf16_to_f64(x)[0]
    for n, (kk, cc) in enumerate(zip(rows, codes)):
        assert u[0, n] == x64[kk] * E2M1[cc] * (4.0 if kk >= 16 else 1.0) * 1.25


def test_gptoss_swiglu_clamps():
    # one nonzero code per column, so u is known exactly: gates 120 and 20 clamp to 7 (min only),
    # linear 120 to 7 and -120 to -7
    K, I = 16, 2
    w = np.zeros((1, K, I), np.uint8)
    w[0, 0, 0] = 0x77            # columns 0 (gate) and 1 (linear) = 6.0 at k = 0
    w[0, 0, 1] = 0xF2            # column 2 (gate) = 1.0, column 3 (linear) = -6.0
    s = np.full((1, 1, 2 * I), 0x38, np.uint8)
    x = synth.to_bf16_bits(np.array([[20.0] + [0.0] * (K - 1)], np.float32))
    g = np.array([1.0], np.float32)
    act = dict(alpha=1.702, beta=1.0, limit=7.0)
    h, u = cpp.fc1_swiglu(x, 1, w, s, g, "nvfp4", np.array([0, 1], np.int32), np.array([0], np.int32), act)
    assert u[0].tolist() == [120.0, 120.0, 20.0, -120.0]
    a, b, lim = 1.702, 1.0, 7.0
    exact = [lim / (1 + np.exp(-a * lim)) * (lim + b), lim / (1 + np.exp(-a * lim)) * (-lim + b)]
    np.testing.assert_array_equal(h[0], codecs.bf16_from_f64(np.array(exact)))


def test_layer_E1_k1_is_dense_swiglu_ffn():
    L = _tiny_layer("nvfp4", seed=6, E=1, T=5, k=1, H=64, I=48)
    r = cpp.layer(L)
    W1 = torch.tensor(table_dequant(L.w1[0], L.s1[0], L.g1[0], "nvfp4"))
    W2 = torch.tensor(table_dequant(L.w2[0], L.s2[0], L.g2[0], "nvfp4"))
    x = torch.tensor(codecs.bf16_to_f64(L.x))
    u = x @ W1
    h = torch.nn.functional.silu(u[:, 0::2]) * u[:, 1::2]
    hb = torch.tensor(codecs.bf16_to_f64(r["h"]))
    torch.testing.assert_close(hb, h, rtol=2 ** -8, atol=1e-30)
    assert np.all(r["w"] == 1.0)
    np.testing.assert_allclose(r["out"], (hb @ W2).numpy(), rtol=1e-12)


def test_finalize_k1_and_identical_rows():
    rng = np.random.default_rng(8)
    y = rng.standard_normal((6, 10))
    np.testing.assert_array_equal(cpp.finalize(y, np.ones((6, 1)), np.arange(6), 6, 1), y)
    yk = np.repeat(rng.standard_normal((1, 10)), 4, axis=0)
    w = scipy.special.softmax(rng.standard_normal(4))[None, :]
    np.testing.assert_allclose(cpp.finalize(yk, w, np.array([2, 0, 3, 1]), 1, 4)[0], yk[0], rtol=1e-15)


@pytest.mark.parametrize("fmt", ["nvfp4", "mxfp4"])
def test_concat_swiglu_equals_interleaved_on_permuted_columns(fmt):
    L = _tiny_layer(fmt, seed=11, E=4, T=4, k=2, H=64, I=32)
    c = L.cfg
    idx, _ = cpp.route_topk(L.logits, c.k)
    off, p2e, _ = cpp.expert_maps(idx, c.E)
    act = dict(alpha=1.702, beta=1.0, limit=7.0)
    hc, uc = cpp.fc1_swiglu(L.x, c.k, L.w1, L.s1, L.g1, fmt, off, p2e, dict(act, fusion=2))
    wi, si = _concat_to_interleaved(L.w1, L.s1)
    hi, ui = cpp.fc1_swiglu(L.x, c.k, wi, si, L.g1, fmt, off, p2e, dict(act, fusion=1))
    np.testing.assert_array_equal(hc, hi)
    np.testing.assert_array_equal(uc[:, :c.I], ui[:, 0::2])
    cols = np.array([0, 5, 31])
    hs, _ = cpp.fc1_swiglu(L.x, c.k, L.w1, L.s1, L.g1, fmt, off, p2e, dict(act, fusion=2), cols=cols)
    np.testing.assert_array_equal(hs[:, cols], hc[:, cols])
    ys = cpp.fc2(hc, L.w2, L.s2, L.g2, fmt, off, cols=cols)
    np.testing.assert_array_equal(ys, cpp.fc2(hc, L.w2, L.s2, L.g2, fmt, off)[:, cols])


# ------------------------------------------- two independent oracles agree --

CROSS = [
    synth.TINY,
    synth.DECODE,
    synth.shrink(synth.MTP8, E=64, T=8, k=8, H=512, I=272, seed=2),
    synth.shrink(synth.MX_DECODE, E=40, T=8, k=8, H=544, I=160, seed=3),
    dataclasses.replace(synth.shrink(synth.MX_DECODE, E=12, T=4, k=4, H=256, I=96, seed=7), mx_global=True),
    synth.shrink(synth.FP8_MTP4, E=24, T=4, k=8, H=256, I=96, seed=8),
]


@pytest.mark.parametrize("cfg", CROSS, ids=[c.name for c in CROSS])
@pytest.mark.parametrize("variant", ["standard", "gptoss_concat", "router_weights"])
def test_cpp_oracle_equals_numpy_oracle(cfg, variant):
    if variant != "standard" and cfg is synth.DECODE:
        pytest.skip("the full decode layer runs once, in the standard variant")
    L = synth.layer_inputs(cfg)
    act = dict(alpha=1.702, beta=1.0, limit=7.0, fusion=2) if variant == "gptoss_concat" else None
    rw = synth.router_weights(cfg) if variant == "router_weights" else None
    a = cpp.layer(L, act=act, router_weights=rw)
    b = moe.layer(L, act=act, router_weights=rw)
    for n in ("idx", "offsets", "p2e", "e2p", "h"):
        np.testing.assert_array_equal(a[n], b[n], err_msg=n)
    for n in ("w", "y", "out"):
        scale = np.sqrt(np.mean(b[n] ** 2, axis=-1, keepdims=True))
        np.testing.assert_array_less(np.abs(a[n] - b[n]), 1e-12 * (np.abs(b[n]) + scale) + 1e-300, err_msg=n)
    np.testing.assert_array_equal(cpp.route_topk(L.logits, cfg.k)[0], route.route_topk(L.logits, cfg.k)[0])
