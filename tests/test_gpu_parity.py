"""GPU parity: the HIP path (through the C ABI) against the float64 oracle.

Bit-exact: routing indices, expert maps, dequantized bf16.  Floating-point
outputs: the oracle.tolerance rule.  Stage-wise checks feed the oracle the
GPU's own previous-stage outputs; end-to-end checks run the oracle from the
inputs alone, taking h's bf16 rounding the GPU's way only where the tests/ties
rule shows it is a float32 rounding tie.  Each case prints its name before it
touches the GPU.
"""
import numpy as np
import pytest
import torch

import synth
from gpu_util import bf16_dev, bf16_host, layer_dev, print_case, to_dev, weights_dev
from ties import h_roundings_differ_only_at_ties
from oracle import codecs, cpp, dequant, moe, route, tolerance

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import fp4_weight_only_amd  # noqa: F401  (raises if the library is not built)


# Shapes the oracle finishes in seconds that still span several tiles, several
# k chunks and ragged tails (N not a multiple of 256, K not of 256).
SMALL = [
    synth.shrink(synth.TINY, seed=0),
    synth.shrink(synth.DECODE, E=37, T=7, k=5, H=320, I=144, seed=1),         # 35 rows, ragged N/K
    synth.shrink(synth.MTP8, E=64, T=8, k=8, H=512, I=272, seed=2),           # 64 rows, hot experts m=8
    synth.shrink(synth.MX_DECODE, E=40, T=8, k=8, H=544, I=160, seed=3),      # MXFP4, ragged
    synth.shrink(synth.DECODE, E=16, T=64, k=1, H=256, I=64, seed=4),         # m up to 64 per expert
    synth.shrink(synth.MX_DECODE, E=4, T=16, k=4, H=1024, I=512, seed=5),     # every expert has 16 rows
    # two k chunks per GEMV workgroup (five chunks: the last pair has one)
    synth.shrink(synth.DECODE, E=16, T=1, k=4, H=1184, I=1040, seed=40),      # one NVFP4 row; FC2's K tail inside a lane
    synth.shrink(synth.MX_DECODE, E=24, T=8, k=8, H=1184, I=1056, seed=41),   # MXFP4, FC1 and FC2 in five chunks
    synth.shrink(synth.MTP4, E=32, T=2, k=8, H=512, I=192, seed=26),          # T=2: one two-row pass
    synth.shrink(synth.MTP4, E=32, T=3, k=8, H=512, I=192, seed=27),          # T=3: 3-row experts over two-row slots (2 + 1)
]
FULL = [synth.TINY, synth.DECODE, synth.MTP4, synth.MTP8]


def run_gpu_layer(L, act=None, path=None, rw=None):
    layer, logits, x = layer_dev(L, act=act, path=path)
    print_case("layer", L.cfg.name, "act", act, "router_weights", rw is not None)
    layer.run(logits, x, router_weights=None if rw is None else to_dev(rw))
    torch.cuda.synchronize()
    return dict(idx=layer.topk_idx.cpu().numpy(), w=layer.topk_w.cpu().numpy().astype(np.float64),
                offsets=layer.offsets.cpu().numpy(), p2e=layer.p2e.cpu().numpy(), e2p=layer.e2p.cpu().numpy(),
                h=bf16_host(layer.h), y=layer.y.cpu().numpy().astype(np.float64),
                out=codecs.bf16_to_f64(bf16_host(layer.out)))


def assert_close(name, gpu, ref):
    ok, rep = tolerance.check(gpu, ref)
    print(name, rep, flush=True)
    assert ok, (name, rep)


def check_layer(L, act=None, cols1=None, cols2=None, path=None, rw=None, orc="numpy"):
    """act: (alpha, beta, limit[, fusion]); rw: router_weights [T][E] or None;
    orc: "numpy" (oracle.route / oracle.moe) or "cpp" (the C++ oracle, same calls)."""
    c = L.cfg
    R, M = (route, moe) if orc == "numpy" else (cpp, cpp)
    g = run_gpu_layer(L, act, path, rw)
    oact = None if act is None else dict(alpha=act[0], beta=act[1], limit=act[2],
                                         fusion=act[3] if len(act) > 3 else 1)
    # routing and maps: bit-exact
    if rw is None:
        idx, wts = R.route_topk(L.logits, c.k)
    else:
        idx, wts = R.route_topk_router_weights(L.logits, rw, c.k)
        assert np.array_equal(g["w"], wts)     # a gather: exact
    off, p2e, e2p = R.expert_maps(idx, c.E)
    assert np.array_equal(g["idx"], idx)
    assert np.array_equal(g["offsets"], off)
    assert np.array_equal(g["p2e"], p2e)
    assert np.array_equal(g["e2p"], e2p)
    assert_close("topk_w", g["w"], wts)
    # FC1 stage (inputs identical to the oracle's)
    h_ref, u_ref = M.fc1_swiglu(L.x, c.k, L.w1, L.s1, L.g1, c.fmt, off, p2e, oact, cols=cols1)
    hsel = slice(None) if cols1 is None else cols1
    assert_close("h", codecs.bf16_to_f64(g["h"])[:, hsel], codecs.bf16_to_f64(h_ref)[:, hsel])
    # FC2 stage, fed the GPU's h
    y_ref = M.fc2(g["h"], L.w2, L.s2, L.g2, c.fmt, off, cols=cols2)
    ysel = slice(None) if cols2 is None else cols2
    assert_close("y", g["y"][:, ysel], y_ref)
    # finalize stage, fed the GPU's y and weights
    out_ref = M.finalize(g["y"], g["w"], g["e2p"], c.T, c.k)
    assert_close("out(stage)", g["out"], out_ref)
    # end to end: the oracle chain from the inputs, with h's rounding taken the
    # GPU's way only where it is a tie (see h_roundings_differ_only_at_ties)
    if cols1 is None and cols2 is None:
        # (after the tie check the GPU's h is that chain's h, so y_ref is its y)
        ties = h_roundings_differ_only_at_ties(L, g["h"], h_ref, u_ref, oact, off, p2e)
        print("h rounding ties", ties, flush=True)
        assert_close("out(e2e)", g["out"], M.finalize(y_ref, wts, e2p, c.T, c.k))
    return g


_ORACLE_FC1 = {}


def oracle_e2e(L, gpu_h, act=None, rw=None, orc="numpy", key=None):
    """The oracle's layer output from the inputs alone (numpy or C++ oracle),
    taking h's bf16 rounding the GPU's way only where the tests/ties rule
    shows a float32 rounding tie; returns (out float64 [T][H], h_ref bits).
    key: cache key for the oracle's routing and FC1 (they depend on the
    inputs only)."""
    c = L.cfg
    R, M = (route, moe) if orc == "numpy" else (cpp, cpp)
    oact = None if act is None else dict(alpha=act[0], beta=act[1], limit=act[2],
                                         fusion=act[3] if len(act) > 3 else 1)
    ck = None if key is None else (key, orc)
    if ck is not None and ck in _ORACLE_FC1:
        idx, wts, off, p2e, e2p, h_ref, u_ref = _ORACLE_FC1[ck]
    else:
        idx, wts = R.route_topk(L.logits, c.k) if rw is None else R.route_topk_router_weights(L.logits, rw, c.k)
        off, p2e, e2p = R.expert_maps(idx, c.E)
        h_ref, u_ref = M.fc1_swiglu(L.x, c.k, L.w1, L.s1, L.g1, c.fmt, off, p2e, oact)
        if ck is not None:
            _ORACLE_FC1[ck] = (idx, wts, off, p2e, e2p, h_ref, u_ref)
    ties = h_roundings_differ_only_at_ties(L, gpu_h, h_ref, u_ref, oact, off, p2e)
    print("h rounding ties", ties, flush=True)
    y_ref = M.fc2(gpu_h, L.w2, L.s2, L.g2, c.fmt, off)
    return M.finalize(y_ref, wts, e2p, c.T, c.k), h_ref


@pytest.mark.parametrize("cfg", SMALL, ids=lambda c: c.name)
def test_layer_small(cfg):
    check_layer(synth.layer_inputs(cfg))


@pytest.mark.parametrize("cfg", FULL, ids=lambda c: c.name)
def test_layer_full(cfg):
    check_layer(synth.layer_inputs(cfg))


@pytest.mark.parametrize("path", ["gemv", "grouped"])
def test_layer_mxfp4_decode_full_sampled(path):
    # the 8-token MXFP4 decode at full size on the GEMV path (AUTO's choice
    # at 64 rows) and on the grouped MFMA kernel (path = GROUPED)
    import fp4_weight_only_amd as q
    L = synth.layer_inputs(synth.MX_DECODE)
    rng = np.random.default_rng(0)
    cols1 = np.sort(rng.choice(L.cfg.I, 160, replace=False))
    cols2 = np.sort(rng.choice(L.cfg.H, 320, replace=False))
    check_layer(L, cols1=cols1, cols2=cols2, path=q.QMOE_PATH_GEMV if path == "gemv" else q.QMOE_PATH_GROUPED)


# Variants: concatenated SwiGLU columns (swiglu_fusion=2), MXFP4 with
# per-expert global scales, DeepSeek-style router weights; each on the GEMV
# path and on the grouped path.
VARIANT_GEMV = synth.shrink(synth.DECODE, E=37, T=7, k=5, H=320, I=144, seed=31)       # 35 rows, ragged
VARIANT_GROUPED = synth.shrink(synth.MX_PREFILL, E=24, T=48, k=4, H=512, I=256, seed=32)
STD, GPTOSS = (1.0, 0.0, float("inf")), (1.702, 1.0, 7.0)


@pytest.mark.parametrize("cfg", [VARIANT_GEMV, synth.shrink(synth.MTP8, E=64, T=8, k=8, H=512, I=272, seed=33),
                                 VARIANT_GROUPED], ids=lambda c: c.name)
@pytest.mark.parametrize("act", [STD, GPTOSS], ids=["std", "gptoss"])
def test_concat_swiglu_layer(cfg, act):
    check_layer(synth.layer_inputs(cfg), act=act + (2,))


def test_concat_swiglu_single_chunk_gemv():
    # K = 256: one k chunk, so the concatenated layout alone forces the
    # partial-sum path
    cfg = synth.shrink(synth.TINY, E=8, T=3, k=2, H=256, I=96, seed=34)
    check_layer(synth.layer_inputs(cfg), act=STD + (2,))


@pytest.mark.parametrize("cfg", [synth.shrink(synth.MX_DECODE, E=40, T=8, k=8, H=544, I=160, seed=35),
                                 VARIANT_GROUPED], ids=lambda c: c.name)
def test_mxfp4_global_scale_layer(cfg):
    import dataclasses
    L = synth.layer_inputs(dataclasses.replace(cfg, mx_global=True, name=cfg.name + "_g"))
    assert L.g1 is not None and L.g2 is not None
    check_layer(L)


@pytest.mark.parametrize("cfg", [VARIANT_GEMV, synth.MTP4, VARIANT_GROUPED], ids=lambda c: c.name)
def test_router_weights_layer(cfg):
    L = synth.layer_inputs(cfg)
    check_layer(L, rw=synth.router_weights(cfg))


@pytest.mark.parametrize("T,E,k", [(1, 256, 8), (8, 256, 8), (40, 200, 6), (512, 256, 8)])
def test_route_router_weights(T, E, k):
    import fp4_weight_only_amd as q
    rng = np.random.default_rng(T + E + k)
    lg = rng.integers(0, 6, (T, E)).astype(np.float32)          # ties too
    rw = rng.random((T, E)).astype(np.float32)
    d = dict(idx=torch.empty((T, k), dtype=torch.int32, device="cuda"),
             w=torch.empty((T, k), dtype=torch.float32, device="cuda"),
             off=torch.empty((E + 1,), dtype=torch.int32, device="cuda"),
             p2e=torch.empty((T * k,), dtype=torch.int32, device="cuda"),
             e2p=torch.empty((T * k,), dtype=torch.int32, device="cuda"))
    print_case("route router_weights", T, E, k)
    q.qmoe_route_topk_router_weights(to_dev(lg), to_dev(rw), k, d["idx"], d["w"], d["off"], d["p2e"], d["e2p"])
    torch.cuda.synchronize()
    idx, w = route.route_topk_router_weights(lg, rw, k)
    assert np.array_equal(d["idx"].cpu().numpy(), idx)
    assert np.array_equal(d["w"].cpu().numpy().astype(np.float64), w)
    off, p2e, e2p = route.expert_maps(idx, E)
    assert np.array_equal(d["off"].cpu().numpy(), off)
    assert np.array_equal(d["p2e"].cpu().numpy(), p2e)
    assert np.array_equal(d["e2p"].cpu().numpy(), e2p)


# FP8 E4M3 weight-only (W8A16): [E][N][K] bytes, per-expert global scale.
FP8_SMALL = [
    synth.shrink(synth.FP8_MTP4, E=37, T=7, k=5, H=320, I=144, seed=41),     # 35 rows, ragged N
    synth.shrink(synth.FP8_MTP4, E=8, T=2, k=2, H=2304, I=96, seed=42),      # K = 2304: two k passes
    synth.shrink(synth.FP8_MTP4, E=16, T=64, k=1, H=256, I=64, seed=43),     # up to 64 rows per expert
    synth.shrink(synth.FP8_MTP4, E=24, T=48, k=4, H=512, I=256, seed=47),    # 192 rows: prefill-sized batch
    synth.shrink(synth.FP8_MTP4, E=8, T=40, k=2, H=1024, I=160, seed=48),    # 80 rows, ragged N, 4 columns per lane row
    synth.with_rows(synth.FP8_MTP4, 1, "fp8_T1"),
    synth.FP8_MTP4,
    synth.with_rows(synth.FP8_MTP4, 8, "fp8_T8"),
]


@pytest.mark.parametrize("cfg", FP8_SMALL, ids=lambda c: c.name)
def test_fp8_layer(cfg):
    check_layer(synth.layer_inputs(cfg))


@pytest.mark.parametrize("act", [STD, GPTOSS], ids=["std", "gptoss"])
def test_fp8_concat_and_gptoss(act):
    cfg = synth.shrink(synth.FP8_MTP4, E=37, T=7, k=5, H=320, I=144, seed=44)
    check_layer(synth.layer_inputs(cfg), act=act + (2,))
    check_layer(synth.layer_inputs(cfg), act=act)


FP8_GROUPED = synth.shrink(synth.FP8_MTP4, E=24, T=48, k=4, H=512, I=256, seed=49)     # 192 rows


@pytest.mark.parametrize("path", ["gemv", "grouped"])
def test_fp8_same_shape_both_paths(path):
    import fp4_weight_only_amd as q
    p = q.QMOE_PATH_GEMV if path == "gemv" else q.QMOE_PATH_GROUPED
    check_layer(synth.layer_inputs(FP8_GROUPED), path=p)


@pytest.mark.parametrize("act", [STD, GPTOSS], ids=["std", "gptoss"])
def test_fp8_grouped_concat_and_gptoss(act):
    check_layer(synth.layer_inputs(FP8_GROUPED), act=act + (2,))
    check_layer(synth.layer_inputs(FP8_GROUPED), act=act)


def test_fp8_grouped_multi_tile():
    # 1024 rows over 64 experts (several 64-row m tiles per expert), K = 1024:
    # a K loop of 16 slices, N = 1024 and 1024: four n tiles
    cfg = synth.dataclasses.replace(synth.shrink(synth.FP8_MTP4, E=64, T=256, k=4, H=1024, I=512, seed=50),
                                    routing="zipf")
    check_layer(synth.layer_inputs(cfg))


@pytest.mark.parametrize("act", [STD, GPTOSS], ids=["std", "gptoss"])
def test_fp8_grouped_half_last_slice(act):
    # K = 576 (FC1) and 192 (FC2): the last 128-k slice holds 64 k; N = 384
    # and 576 end in part-filled n tiles
    import fp4_weight_only_amd as q
    cfg = synth.shrink(synth.FP8_MTP4, E=16, T=48, k=4, H=576, I=192, seed=51)
    check_layer(synth.layer_inputs(cfg), path=q.QMOE_PATH_GROUPED, act=act)
    check_layer(synth.layer_inputs(cfg), path=q.QMOE_PATH_GROUPED, act=act + (2,))


def test_fp8_every_finite_byte_through_the_gemv():
    # every finite E4M3 byte at every lane position of a 16-byte load
    cfg = synth.shrink(synth.FP8_MTP4, E=2, T=2, k=1, H=512, I=128, seed=45)
    L = synth.layer_inputs(cfg)
    finite = np.array([b for b in range(256) if (b & 0x7F) != 0x7F], np.uint8)
    for w in (L.w1, L.w2):
        E, N, K = w.shape
        w[:] = finite[(np.arange(E * N * K).reshape(E, N, K) * 7 + np.arange(N)[None, :, None] * 3) % len(finite)]
        assert set(np.unique(w)) == set(finite)
    L.x[:] = synth.to_bf16_bits(np.full(L.x.shape, 0.01, np.float32))   # keep SwiGLU finite with 448-sized weights
    check_layer(L)


def test_fp8_dequant_every_byte():
    import fp4_weight_only_amd as q
    E, N, K = 3, 96, 160
    rng = np.random.default_rng(46)
    w = rng.integers(0, 256, (E, N, K), dtype=np.uint8)
    w[0].reshape(-1)[:256] = np.arange(256)
    g = np.array([1.0, 0.37, 1.9], np.float32)
    out = torch.empty((E, N, K), dtype=torch.int16, device="cuda")
    print_case("fp8 dequant", E, N, K)
    q.qmoe_dequant_fp8(q.FP8Weights(to_dev(w), to_dev(g)), out)
    torch.cuda.synchronize()
    got = out.cpu().numpy().view(np.uint16)
    ref = dequant.dequant_fp8_bf16(w, g)
    nan = (w & 0x7F) == 0x7F
    assert np.all((got[nan] & 0x7F80) == 0x7F80) and np.all((got[nan] & 0x7F) != 0)   # NaN
    assert np.array_equal(got[~nan], ref[~nan])


def test_gptoss_swiglu_variant():
    cfg = synth.shrink(synth.DECODE, E=16, T=4, k=4, H=256, I=128, seed=7)
    L = synth.layer_inputs(cfg)
    check_layer(L, act=(1.702, 1.0, 7.0))


def test_route_ties_and_signed_zero():
    import fp4_weight_only_amd as q
    lg = np.zeros((6, 256), np.float32)
    lg[0, :] = 0.0
    lg[1, ::2] = -0.0
    lg[2, [5, 9, 200, 3]] = 2.5
    lg[3, :] = np.float32(-1e30)
    lg[3, 255] = np.float32(-np.inf)
    lg[4, :] = np.arange(256, dtype=np.float32)[::-1] * 0 + 1.0
    lg[5, 17] = np.inf
    T, E, k = lg.shape[0], 256, 8
    d = dict(idx=torch.empty((T, k), dtype=torch.int32, device="cuda"),
             w=torch.empty((T, k), dtype=torch.float32, device="cuda"),
             off=torch.empty((E + 1,), dtype=torch.int32, device="cuda"),
             p2e=torch.empty((T * k,), dtype=torch.int32, device="cuda"),
             e2p=torch.empty((T * k,), dtype=torch.int32, device="cuda"))
    print_case("route ties")
    q.qmoe_route_topk(to_dev(lg), k, d["idx"], d["w"], d["off"], d["p2e"], d["e2p"])
    torch.cuda.synchronize()
    idx, w = route.route_topk(lg, k)
    assert np.array_equal(d["idx"].cpu().numpy(), idx)
    gw = d["w"].cpu().numpy()
    fin = np.isfinite(w)
    np.testing.assert_allclose(gw[:5], w[:5], rtol=1e-6)
    off, p2e, e2p = route.expert_maps(idx, E)
    assert np.array_equal(d["off"].cpu().numpy(), off)
    assert np.array_equal(d["p2e"].cpu().numpy(), p2e)
    assert fin[:5].all()


@pytest.mark.parametrize("T,E,k", [(1, 1, 1), (3, 5, 5), (512, 256, 8), (100, 200, 3), (4096, 256, 1)])
def test_route_shapes(T, E, k):
    import fp4_weight_only_amd as q
    rng = np.random.default_rng(T * 7 + E)
    lg = rng.standard_normal((T, E)).astype(np.float32)
    lg[:, rng.integers(0, E, 3)] += 1.0  # some duplicates and skew
    d = dict(idx=torch.empty((T, k), dtype=torch.int32, device="cuda"),
             w=torch.empty((T, k), dtype=torch.float32, device="cuda"),
             off=torch.empty((E + 1,), dtype=torch.int32, device="cuda"),
             p2e=torch.empty((T * k,), dtype=torch.int32, device="cuda"),
             e2p=torch.empty((T * k,), dtype=torch.int32, device="cuda"))
    print_case("route", T, E, k)
    q.qmoe_route_topk(to_dev(lg), k, d["idx"], d["w"], d["off"], d["p2e"], d["e2p"])
    torch.cuda.synchronize()
    idx, w = route.route_topk(lg, k)
    assert np.array_equal(d["idx"].cpu().numpy(), idx)
    assert_close("topk_w", d["w"].cpu().numpy(), w)
    off, p2e, e2p = route.expert_maps(idx, E)
    assert np.array_equal(d["off"].cpu().numpy(), off)
    assert np.array_equal(d["p2e"].cpu().numpy(), p2e)
    assert np.array_equal(d["e2p"].cpu().numpy(), e2p)


@pytest.mark.parametrize("T,E,k", [(1, 256, 8), (4, 256, 8), (8, 256, 8), (9, 256, 8), (16, 200, 8),
                                   (40, 256, 8), (16, 256, 2)])
def test_route_discrete_logits(T, E, k):
    """Logits from four values: nearly every selection round meets equal
    maxima in several lanes (lower expert index wins), and the expert maps
    see few distinct experts with many rows each."""
    import fp4_weight_only_amd as q
    rng = np.random.default_rng(T * 131 + E + k)
    lg = rng.integers(0, 4, (T, E)).astype(np.float32) - 1.5
    d = dict(idx=torch.empty((T, k), dtype=torch.int32, device="cuda"),
             w=torch.empty((T, k), dtype=torch.float32, device="cuda"),
             off=torch.empty((E + 1,), dtype=torch.int32, device="cuda"),
             p2e=torch.empty((T * k,), dtype=torch.int32, device="cuda"),
             e2p=torch.empty((T * k,), dtype=torch.int32, device="cuda"))
    print_case("route discrete", T, E, k)
    q.qmoe_route_topk(to_dev(lg), k, d["idx"], d["w"], d["off"], d["p2e"], d["e2p"])
    torch.cuda.synchronize()
    idx, w = route.route_topk(lg, k)
    assert np.array_equal(d["idx"].cpu().numpy(), idx)
    assert_close("topk_w", d["w"].cpu().numpy(), w)
    off, p2e, e2p = route.expert_maps(idx, E)
    assert np.array_equal(d["off"].cpu().numpy(), off)
    assert np.array_equal(d["p2e"].cpu().numpy(), p2e)
    assert np.array_equal(d["e2p"].cpu().numpy(), e2p)


@pytest.mark.parametrize("fmt", ["nvfp4", "mxfp4"])
def test_every_code_in_every_nibble_through_the_gemv(fmt):
    """Closed form: one nonzero code per column, so u = x_k * e2m1 * scale * g exactly."""
    import fp4_weight_only_amd as q
    from fp4_weight_only_amd.layer import MoELayer
    B = 16 if fmt == "nvfp4" else 32
    K, N = 256, 512
    rng = np.random.default_rng(11)
    w = np.zeros((1, K, N // 2), np.uint8)
    rows = rng.integers(0, K, N)
    codes = np.arange(N) % 16                        # every code in every nibble position
    for n in range(N):
        w[0, rows[n], n // 2] |= np.uint8(codes[n] << (4 * (n % 2)))
    if fmt == "nvfp4":
        s = np.full((1, K // B, N), 0x38, np.uint8)  # 1.0
        g = np.array([0.75], np.float32)
    else:
        s = np.full((1, K // B, N), 127, np.uint8)
        g = None
    x = synth.to_bf16_bits((rng.standard_normal((1, K)) * 3).astype(np.float32))
    wd = weights_dev(w, s, g, fmt)
    w2 = weights_dev(np.zeros((1, N // 2, 16), np.uint8), np.full((1, N // 2 // B, 32), 0x38 if fmt == "nvfp4" else 127, np.uint8),
                     g, fmt)
    layer = MoELayer(1, 1, 1, 32, N // 2, wd, w2)
    print_case("closed form", fmt)
    layer.route(to_dev(np.zeros((1, 1), np.float32)))
    layer.fc1(bf16_dev(x))
    torch.cuda.synchronize()
    h = codecs.bf16_to_f64(bf16_host(layer.h))[0]
    x64 = codecs.bf16_to_f64(x)[0]
    u = x64[rows] * codecs.e2m1_value(codes) * (0.75 if fmt == "nvfp4" else 1.0)
    u32 = u.astype(np.float32).astype(np.float64)   # the exact product rounded once
    href = codecs.bf16_from_f64(moe.swiglu(u32[0::2], u32[1::2]))
    got = bf16_host(layer.h)[0]
    # products are exact; only SwiGLU's exp differs from float64 in the last float32 bits.
    # Values are compared (a gate of -0 summed onto a +0 accumulator is +0: same value).
    ok, rep = tolerance.check(h, codecs.bf16_to_f64(href))
    assert ok, rep
    diff = codecs.bf16_to_f64(got) != codecs.bf16_to_f64(href)
    assert np.count_nonzero(diff) <= 2, np.nonzero(diff)


def _scale_exponent(fmt, byte):
    """floor(log2 |scale|) of a scale byte, from the oracle's codec."""
    v = (codecs.e4m3fn_value if fmt == "nvfp4" else codecs.e8m0_value)(np.array([byte]))[0]
    return 0 if v == 0 else int(np.floor(np.log2(abs(v))))     # E4M3 0x00 / 0x80: a zero scale


def _scale_byte_case(fmt, path, K, N, seed):
    """Weights with one nonzero code per column n (row n of K) whose block
    scale is the byte under test; every scale byte of the codec appears in
    some column (NaN bytes excepted).  The activation of row n is a power of
    two that brings x * code * scale near 1, so products stay exact and
    normal in float32.  On the grouped path (weights formed in bf16) the
    codes at E8M0 bytes 253 and 254 are kept small enough for bf16's range."""
    B = 16 if fmt == "nvfp4" else 32
    rng = np.random.default_rng(seed)
    if fmt == "nvfp4":
        bytes_ = np.array([b for b in range(256) if (b & 0x7F) != 0x7F])
    else:
        bytes_ = np.arange(255)
    assert K >= N
    col_byte = bytes_[(np.arange(N) * 7 + seed) % len(bytes_)]
    assert set(col_byte) == set(bytes_) or N < len(bytes_)
    nonzero = np.array([c for c in range(16) if c not in (0, 8)])
    codes = nonzero[rng.integers(0, len(nonzero), N)]
    if fmt == "mxfp4" and path == "grouped":
        small3 = np.array([1, 2, 3, 4, 5, 9, 10, 11, 12, 13])     # |value| <= 3
        small15 = np.array([1, 2, 3, 9, 10, 11])                  # |value| <= 1.5
        m253, m254 = col_byte == 253, col_byte == 254
        codes[m253] = small3[rng.integers(0, len(small3), m253.sum())]
        codes[m254] = small15[rng.integers(0, len(small15), m254.sum())]
    w = np.zeros((1, K, N // 2), np.uint8)
    s = np.full((1, K // B, N), 0x38 if fmt == "nvfp4" else 127, np.uint8)
    xexp = np.zeros(K, np.int64)
    for n in range(N):
        w[0, n, n // 2] |= np.uint8(codes[n] << (4 * (n % 2)))
        s[0, n // B, n] = col_byte[n]
        xexp[n] = int(np.clip(-_scale_exponent(fmt, col_byte[n]) + rng.integers(-2, 3), -120, 120))
    sign = np.where(rng.random(K) < 0.5, -1.0, 1.0)
    act = synth.to_bf16_bits((sign * np.ldexp(1.0, xexp)).astype(np.float32))[None, :]
    g = np.array([0.75], np.float32) if fmt == "nvfp4" else None
    return w, s, g, act, col_byte


@pytest.mark.parametrize("path", ["gemv", "grouped"])
@pytest.mark.parametrize("fmt", ["nvfp4", "mxfp4"])
def test_every_scale_byte_through_fc1_and_fc2(fmt, path):
    """Every E4M3 byte but the NaN pair (subnormals included) and every E8M0
    byte 0..254 reach FC1 and FC2 as block scales, on the GEMV and the grouped
    kernel, against the oracle; FC2 with one product per output is exact."""
    import fp4_weight_only_amd as q
    p = q.QMOE_PATH_GEMV if path == "gemv" else q.QMOE_PATH_GROUPED
    offsets = to_dev(np.array([0, 1], np.int32))
    p2e = to_dev(np.array([0], np.int32))
    # FC1: K = 512, N = 512 (I = 256): h = SwiGLU(u[2j], u[2j+1])
    K1, N1 = 512, 512
    w1, s1, g1, x, b1 = _scale_byte_case(fmt, path, K1, N1, seed=71)
    wd1 = weights_dev(w1, s1, g1, fmt)
    h = torch.empty((1, N1 // 2), dtype=torch.bfloat16, device="cuda")
    ws = q.alloc_workspace(max(q.fc_workspace_bytes(1, 1, 1, wd1, p), 1 << 16))
    print_case("scale bytes fc1", fmt, path)
    q.qmoe_fp4_gemv_fc1_swiglu(bf16_dev(x), 1, wd1, offsets, p2e, h, ws, path=p)
    torch.cuda.synchronize()
    h_ref, _ = moe.fc1_swiglu(x, 1, w1, s1, g1, fmt, np.array([0, 1]), np.array([0]))
    assert_close("h (every scale byte)", codecs.bf16_to_f64(bf16_host(h)), codecs.bf16_to_f64(h_ref))
    # FC2: K = I = 512 rows, N = H = 256 columns; the input row plays x's part
    K2, N2 = 512, 256
    w2, s2, g2, hin, b2 = _scale_byte_case(fmt, path, K2, N2, seed=72)
    wd2 = weights_dev(w2, s2, g2, fmt)
    y = torch.empty((1, N2), dtype=torch.float32, device="cuda")
    ws2 = q.alloc_workspace(max(q.fc_workspace_bytes(2, 1, 1, wd2, p), 1 << 16))
    print_case("scale bytes fc2", fmt, path)
    q.qmoe_fp4_gemv_fc2(bf16_dev(hin), 1, 1, wd2, offsets, y, ws2, path=p)
    torch.cuda.synchronize()
    y_ref = moe.fc2(hin, w2, s2, g2, fmt, np.array([0, 1]))
    got = y.cpu().numpy().astype(np.float64)
    bad = np.nonzero(got != y_ref)[1]
    assert bad.size == 0, [(int(n), int(b2[n]), got[0, n], y_ref[0, n]) for n in bad[:8]]
    seen = set(b1) | set(b2)
    expect = set(range(255)) if fmt == "mxfp4" else {b for b in range(256) if (b & 0x7F) != 0x7F}
    assert seen == expect


FUSED = [
    synth.TINY,
    synth.shrink(synth.DECODE, E=37, T=7, k=5, H=320, I=144, seed=1),      # ragged K/N, several k chunks
    synth.MTP4,
    synth.MTP8,
    synth.shrink(synth.MX_DECODE, E=40, T=8, k=8, H=544, I=160, seed=3),
    synth.shrink(synth.MX_PREFILL, E=16, T=64, k=4, H=512, I=256, seed=21),  # grouped path
]


@pytest.mark.parametrize("cfg", FUSED, ids=lambda c: c.name)
def test_fc2_finalize_fused_equals_separate_calls(cfg):
    """qmoe_fp4_gemv_fc2_finalize adds FC2's partial sums per routed row in the
    order the split-K epilogue does, then weights them as qmoe_finalize does:
    the output must equal the separate calls bit for bit, with its output and
    workspace poisoned first, and match the oracle's end-to-end output."""
    L = synth.layer_inputs(cfg)
    layer, logits, x = layer_dev(L)
    print_case("fused fc2+finalize", cfg.name)
    layer.run(logits, x)
    torch.cuda.synchronize()
    ref = bf16_host(layer.out).copy()
    gpu_h = bf16_host(layer.h).copy()
    layer.out.view(torch.int16).fill_(0x7FC1)   # poison
    layer.ws.view(torch.int16).fill_(0x7FC1)
    layer.fc2_finalize()
    torch.cuda.synchronize()
    got = bf16_host(layer.out)
    assert np.array_equal(got, ref)
    # and the fused output itself against the oracle's end-to-end output
    out_ref, _ = oracle_e2e(L, gpu_h)
    assert_close("fused out vs oracle", codecs.bf16_to_f64(got), out_ref)


ROUTE_FC1 = [
    synth.shrink(synth.TINY, seed=0),
    synth.shrink(synth.DECODE, E=37, T=7, k=5, H=320, I=144, seed=1),      # 35 rows; two tokens per wave
    synth.shrink(synth.DECODE, E=20, T=5, k=3, H=128, I=64, seed=22),      # K = 128: two waves per workgroup
    synth.shrink(synth.MTP8, E=64, T=8, k=8, H=512, I=272, seed=2),        # 64 rows (the limit)
    synth.shrink(synth.DECODE, E=16, T=64, k=1, H=256, I=64, seed=4),      # 64 tokens, k = 1, one k chunk
    synth.shrink(synth.MX_DECODE, E=40, T=8, k=8, H=544, I=160, seed=3),   # MXFP4
    synth.shrink(synth.MTP4, T=16, k=4, H=512, I=128, seed=23),            # E = 256, 16 tokens
    synth.DECODE,
    synth.MTP4,
]


@pytest.mark.parametrize("mode", ["softmax", "router_weights", "gptoss_concat"])
@pytest.mark.parametrize("cfg", ROUTE_FC1, ids=lambda c: c.name)
def test_route_fc1_equals_separate_calls(cfg, mode):
    """qmoe_fp4_route_fc1_swiglu runs the routing of all tokens in every FC1
    workgroup: every output (selections, weights, maps, h) must equal the
    separate routing and FC1 GEMV calls bit for bit, and h must match the
    oracle's FC1."""
    import fp4_weight_only_amd as q
    L = synth.layer_inputs(cfg)
    act = GPTOSS + (q.QMOE_SWIGLU_CONCAT,) if mode == "gptoss_concat" else None
    layer, logits, x = layer_dev(L, act=act, path=q.QMOE_PATH_GEMV)
    rw = to_dev(synth.router_weights(cfg)) if mode == "router_weights" else None
    print_case("route+fc1", cfg.name, mode)
    outs = (layer.topk_idx, layer.topk_w, layer.offsets, layer.p2e, layer.e2p, layer.h)
    layer.route(logits, rw)
    layer.fc1(x)
    torch.cuda.synchronize()
    ref = [t.view(torch.int32 if t.element_size() == 4 else torch.int16).cpu().numpy().copy() for t in outs]
    for t in outs:                                   # poison every output
        t.view(torch.int32 if t.element_size() == 4 else torch.int16).fill_(-7)
    layer.route_fc1(logits, x, rw)
    torch.cuda.synchronize()
    for name, t, r in zip(("idx", "w", "offsets", "p2e", "e2p", "h"), outs, ref):
        got = t.view(torch.int32 if t.element_size() == 4 else torch.int16).cpu().numpy()
        assert np.array_equal(got, r), name
    # the fused call's h against the oracle's FC1 (routing compared bit for bit)
    rwh = None if rw is None else synth.router_weights(cfg)
    idx, _ = (route.route_topk(L.logits, cfg.k) if rwh is None
              else route.route_topk_router_weights(L.logits, rwh, cfg.k))
    assert np.array_equal(layer.topk_idx.cpu().numpy(), idx)
    _, h_ref = oracle_e2e(L, bf16_host(layer.h), act, rwh, key=(cfg.name, mode))
    assert_close("fused h vs oracle", codecs.bf16_to_f64(bf16_host(layer.h)), codecs.bf16_to_f64(h_ref))


LAYER_DECODE = ROUTE_FC1 + SMALL[-2:] + [
    synth.shrink(synth.DECODE, E=8, T=2, k=2, H=2304, I=96, seed=24),      # FC1 in 9 k chunks; FC2 K = 96 < its chunk
    synth.shrink(synth.MX_DECODE, E=12, T=16, k=4, H=1024, I=256, seed=25),  # MXFP4, experts with > 4 rows
]


@pytest.mark.parametrize("route_in_fc1", [0, 1])
@pytest.mark.parametrize("mode", ["softmax", "router_weights", "gptoss_concat"])
@pytest.mark.parametrize("cfg", LAYER_DECODE, ids=lambda c: c.name)
def test_layer_decode_equals_separate_calls(cfg, mode, route_in_fc1):
    """qmoe_fp4_moe_layer_decode forms h inside FC2's staging from FC1's
    partial sums: the routing outputs and out must equal the separate routing,
    FC1 (GEMV) and fused FC2 + finalize (GEMV) calls bit for bit (outputs and
    workspace poisoned first), and out must match the oracle's end-to-end
    output."""
    import fp4_weight_only_amd as q
    L = synth.layer_inputs(cfg)
    act = GPTOSS + (q.QMOE_SWIGLU_CONCAT,) if mode == "gptoss_concat" else None
    layer, logits, x = layer_dev(L, act=act, path=q.QMOE_PATH_GEMV)
    rw = to_dev(synth.router_weights(cfg)) if mode == "router_weights" else None
    print_case("layer decode", cfg.name, mode, "route_in_fc1", route_in_fc1)
    outs = (layer.topk_idx, layer.topk_w, layer.offsets, layer.p2e, layer.e2p, layer.out)
    layer.route(logits, rw)
    layer.fc1(x)
    layer.fc2_finalize()
    torch.cuda.synchronize()
    ref = [t.view(torch.int32 if t.element_size() == 4 else torch.int16).cpu().numpy().copy() for t in outs]
    gpu_h = bf16_host(layer.h).copy()
    for t in outs:                                   # poison every output and the workspace
        t.view(torch.int32 if t.element_size() == 4 else torch.int16).fill_(-7)
    layer.ws.view(torch.int16).fill_(0x7FC1)
    layer.decode_layer(logits, x, rw, route_in_fc1=bool(route_in_fc1))
    torch.cuda.synchronize()
    for name, t, r in zip(("idx", "w", "offsets", "p2e", "e2p", "out"), outs, ref):
        got = t.view(torch.int32 if t.element_size() == 4 else torch.int16).cpu().numpy()
        assert np.array_equal(got, r), name
    # the whole-layer call's output against the oracle's end-to-end output
    rwh = None if rw is None else synth.router_weights(cfg)
    out_ref, _ = oracle_e2e(L, gpu_h, act, rwh, key=(cfg.name, mode))
    assert_close("layer decode out vs oracle", codecs.bf16_to_f64(bf16_host(layer.out)), out_ref)


PERSISTENT = LAYER_DECODE + [synth.MTP8, synth.shrink(synth.MX_DECODE, E=32, T=8, k=8, H=1024, I=512, seed=28),
                             synth.shrink(synth.MTP4, E=64, T=6, k=8, H=2304, I=1280, seed=29),
                             # separate FC1 calls on the two-chunk GEMV, five k chunks
                             synth.shrink(synth.MX_DECODE, E=24, T=8, k=8, H=1184, I=1024, seed=42),
                             synth.shrink(synth.DECODE, E=16, T=1, k=4, H=1184, I=256, seed=43)]


@pytest.mark.parametrize("mode", ["softmax", "router_weights", "gptoss_concat"])
@pytest.mark.parametrize("cfg", PERSISTENT, ids=lambda c: c.name)
def test_layer_persistent(cfg, mode):
    """qmoe_fp4_moe_layer_persistent runs the whole layer in one launch: the
    routing outputs and out must equal the separate routing, FC1 (GEMV) and
    fused FC2 + finalize (GEMV) calls bit for bit, on two calls in a row with
    outputs and the non-counter workspace poisoned before each; the counters
    must be back at zero with the error word clear; and out must match the
    oracle's end-to-end output."""
    import fp4_weight_only_amd as q
    L = synth.layer_inputs(cfg)
    act = GPTOSS + (q.QMOE_SWIGLU_CONCAT,) if mode == "gptoss_concat" else None
    layer, logits, x = layer_dev(L, act=act, path=q.QMOE_PATH_GEMV)
    rw = to_dev(synth.router_weights(cfg)) if mode == "router_weights" else None
    print_case("layer persistent", cfg.name, mode)
    if mode == "gptoss_concat" and cfg.I % 256 != 0:
        assert not layer.layer_persistent
        with pytest.raises(q.QmoeError) as ei:
            q.layer_persistent_workspace_bytes(cfg.T, cfg.k, layer.w1, layer.w2, act)
        assert ei.value.status == q.QMOE_EUNSUPPORTED
        return
    assert layer.layer_persistent
    outs = (layer.topk_idx, layer.topk_w, layer.offsets, layer.p2e, layer.e2p, layer.out)
    layer.route(logits, rw)
    layer.fc1(x)
    layer.fc2_finalize()
    torch.cuda.synchronize()
    ref = [t.view(torch.int32 if t.element_size() == 4 else torch.int16).cpu().numpy().copy() for t in outs]
    gpu_h = bf16_host(layer.h).copy()
    for rep in range(2):
        for t in outs:
            t.view(torch.int32 if t.element_size() == 4 else torch.int16).fill_(-7)
        fill_pattern(layer.ws_layer[q.LAYER_SYNC_BYTES:], 0x7FC00001 + rep)
        layer.persistent_layer(logits, x, rw)
        torch.cuda.synchronize()
        for name, t, r in zip(("idx", "w", "offsets", "p2e", "e2p", "out"), outs, ref):
            got = t.view(torch.int32 if t.element_size() == 4 else torch.int16).cpu().numpy()
            assert np.array_equal(got, r), (rep, name)
        assert layer_sync_clean(layer.ws_layer), rep
    rwh = None if rw is None else synth.router_weights(cfg)
    out_ref, _ = oracle_e2e(L, gpu_h, act, rwh, key=(cfg.name, mode))
    assert_close("persistent out vs oracle", codecs.bf16_to_f64(bf16_host(layer.out)), out_ref)


def test_layer_persistent_graph_replay():
    """The one-launch layer captured in a HIP graph over two weight copies
    (the bench's launch path) and replayed three times, with eager calls and
    synchronisations in between: every replay's outputs equal the eager calls'
    bit for bit, and the counters stay at zero."""
    import fp4_weight_only_amd as q
    cfg = synth.shrink(synth.MTP4, E=64, T=4, k=8, H=512, I=256, seed=41)
    L = synth.layer_inputs(cfg)
    layer, logits, x = layer_dev(L, path=q.QMOE_PATH_GEMV)
    print_case("layer persistent graph", cfg.name)
    assert layer.layer_persistent
    wa = (layer.w1, layer.w2)
    wb = tuple(q.FP4Weights(w.w.clone(), w.scales.clone(), None if w.gscale is None else w.gscale * 0.5, w.fmt)
               for w in wa)
    refs = []
    for w in (wa, wb):
        layer.set_weights(*w)
        layer.persistent_layer(logits, x)
        torch.cuda.synchronize()
        refs.append(bf16_host(layer.out).copy())
    assert not np.array_equal(refs[0], refs[1])
    outs = [torch.empty_like(layer.out) for _ in range(2)]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())

    def body():
        for i, w in enumerate((wa, wb)):
            layer.set_weights(*w)
            layer.persistent_layer(logits, x)
            outs[i].copy_(layer.out)

    with torch.cuda.stream(s):
        body()   # warm-up outside the capture
    s.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        body()
    for rep in range(3):
        for o in outs:
            o.view(torch.int16).fill_(-7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i in range(2):
            assert np.array_equal(bf16_host(outs[i]), refs[i]), (rep, i)
        assert layer_sync_clean(layer.ws_layer), rep
        layer.set_weights(*wa)      # eager work between replays
        layer.route(logits)
        layer.fc1(x)
        layer.fc2_finalize()
        torch.cuda.synchronize()
        assert np.array_equal(bf16_host(layer.out), refs[0]), rep


def test_layer_persistent_wait_bound(monkeypatch):
    """A wait that runs out sets the error word and the call still completes:
    with the bound lowered to 0 (QMOE_LAYER_MAX_POLLS), the FC2 items of a
    one-round layer poll before FC1 has finished and give up at once.  After
    the workspace is zeroed again the next call is exact."""
    import fp4_weight_only_amd as q
    L = synth.layer_inputs(synth.TINY)
    layer, logits, x = layer_dev(L, path=q.QMOE_PATH_GEMV)
    print_case("layer persistent wait bound", L.cfg.name)
    layer.route(logits)
    layer.fc1(x)
    layer.fc2_finalize()
    torch.cuda.synchronize()
    ref = bf16_host(layer.out).copy()
    monkeypatch.setenv("QMOE_LAYER_MAX_POLLS", "0")
    layer.persistent_layer(logits, x)
    torch.cuda.synchronize()
    assert q.layer_error_word(layer.ws_layer) & 1
    monkeypatch.delenv("QMOE_LAYER_MAX_POLLS")
    layer.ws_layer.zero_()
    layer.out.view(torch.int16).fill_(-7)
    layer.persistent_layer(logits, x)
    torch.cuda.synchronize()
    assert q.layer_error_word(layer.ws_layer) == 0
    assert np.array_equal(bf16_host(layer.out), ref)
    assert layer_sync_clean(layer.ws_layer)


def test_layer_persistent_mxfp4_decode_full():
    """The 8-token MXFP4 layer (E=256, hidden 4096, intermediate 2048) in one
    launch: bit for bit the separate GEMV calls; FC2 + finalize against the
    oracle on sampled columns, fed the GPU's h (the separate FC1 call's h is
    checked against the oracle by test_layer_mxfp4_decode_full_sampled)."""
    import fp4_weight_only_amd as q
    L = synth.layer_inputs(synth.MX_DECODE)
    c = L.cfg
    layer, logits, x = layer_dev(L, path=q.QMOE_PATH_GEMV)
    print_case("layer persistent", c.name)
    assert layer.layer_persistent
    layer.route(logits)
    layer.fc1(x)
    layer.fc2_finalize()
    torch.cuda.synchronize()
    ref = bf16_host(layer.out).copy()
    gpu_h = bf16_host(layer.h).copy()
    layer.out.view(torch.int16).fill_(-7)
    layer.persistent_layer(logits, x)
    torch.cuda.synchronize()
    assert np.array_equal(bf16_host(layer.out), ref)
    assert layer_sync_clean(layer.ws_layer)
    rng = np.random.default_rng(3)
    cols = np.sort(rng.choice(c.H, 256, replace=False))
    idx, wts = route.route_topk(L.logits, c.k)
    off, p2e, e2p = route.expert_maps(idx, c.E)
    y_ref = moe.fc2(gpu_h, L.w2, L.s2, L.g2, c.fmt, off, cols=cols)
    assert_close("persistent out vs oracle (sampled)", codecs.bf16_to_f64(ref)[:, cols],
                 moe.finalize(y_ref, wts, e2p, c.T, c.k))


@pytest.mark.parametrize("K", [512, 384], ids=["lds_tile", "direct_128x512"])
@pytest.mark.parametrize("fmt", ["nvfp4", "mxfp4", "mxfp4_g"])
def test_dequant_small_exhaustive_scales(fmt, K):
    """Every scale byte (NaN bytes aside) with random codes; MXFP4 with and
    without a global scale (the two take different conversion paths); K = 512
    runs the LDS-staged kernel, K = 384 the direct kernel's 128 x 512 tile."""
    import fp4_weight_only_amd as q
    with_g = fmt == "mxfp4_g"
    fmt = "mxfp4" if with_g else fmt
    B = 16 if fmt == "nvfp4" else 32
    E, N = 2, 256 * 2
    rng = np.random.default_rng(12)
    w = synth.packed_codes(synth.stream(1, 2), (E, K, N // 2))
    s = (np.arange(E * (K // B) * N) % 256).astype(np.uint8).reshape(E, K // B, N)   # every scale byte
    if fmt == "nvfp4":
        s[s == 0x7F] = 0x38
        s[s == 0xFF] = 0xB8
        g = np.array([1.3, 0.6], np.float32)
    else:
        s[s == 255] = 127
        g = np.array([1.3, 0.6], np.float32) if with_g else None
    out = torch.empty((E, N, K), dtype=torch.bfloat16, device="cuda")
    print_case("dequant small", fmt, "g" if g is not None else "")
    q.qmoe_dequant_fp4(weights_dev(w, s, g, fmt), out)
    torch.cuda.synchronize()
    ref = dequant.dequant_bf16(w, s, g, fmt)
    assert np.array_equal(bf16_host(out), ref)
    _ = rng


@pytest.mark.parametrize("fmt", ["nvfp4", "mxfp4"])
@pytest.mark.parametrize("K,N", [(512, 256), (384, 512), (320, 512), (384, 256), (320, 256)])
def test_dequant_tile_shapes(fmt, K, N):
    """One shape per dequant kernel branch: the LDS-staged 256 x 256 tile (K %
    256 == 0), then the direct kernel's tiles 128 k x 512 n (K % 128 == 0, N %
    512 == 0), 64 x 512 (N % 512 == 0), 128 x 256 (K % 128 == 0) and 64 x 256."""
    import fp4_weight_only_amd as q
    B = 16 if fmt == "nvfp4" else 32
    E = 3
    w = synth.packed_codes(synth.stream(2, 2), (E, K, N // 2))
    if fmt == "nvfp4":
        s = synth.e4m3_scales(synth.stream(2, 3), (E, K // B, N))
        g = synth.global_scales(synth.stream(2, 4), E)
    else:
        s = synth.e8m0_scales(synth.stream(2, 3), (E, K // B, N))
        g = None
    out = torch.empty((E, N, K), dtype=torch.bfloat16, device="cuda")
    print_case("dequant shape", fmt, K, N)
    q.qmoe_dequant_fp4(weights_dev(w, s, g, fmt), out)
    torch.cuda.synchronize()
    assert np.array_equal(bf16_host(out), dequant.dequant_bf16(w, s, g, fmt))


def test_dequant_full_config():
    import fp4_weight_only_amd as q
    c = synth.DEQUANT
    w, s, g = synth.dequant_inputs(c)
    out = torch.empty((c.E, c.N, c.K), dtype=torch.bfloat16, device="cuda")
    print_case("dequant full", c.name)
    q.qmoe_dequant_fp4(weights_dev(w, s, g, c.fmt), out)
    torch.cuda.synchronize()
    got = bf16_host(out)
    for e in range(c.E):                       # expert by expert to bound host memory
        ref = dequant.dequant_bf16(w[e:e + 1], s[e:e + 1], None, c.fmt)[0]
        assert np.array_equal(got[e], ref), e


def test_gemv_window_and_paths():
    import fp4_weight_only_amd as q
    cfg = synth.shrink(synth.DECODE, E=32, T=8, k=8, H=256, I=64, seed=9)
    L = synth.layer_inputs(cfg)
    check_layer(L)                                       # 64 rows: GEMV window edge
    cfg65 = synth.shrink(synth.DECODE, E=32, T=13, k=5, H=256, I=64, seed=9)   # 65 rows
    L65 = synth.layer_inputs(cfg65)
    c = L65.cfg
    w1 = weights_dev(L65.w1, L65.s1, L65.g1, c.fmt)
    with pytest.raises(q.QmoeError) as ei:          # the size query already refuses 65 rows on GEMV
        q.fc_workspace_bytes(1, c.T, c.k, w1, q.QMOE_PATH_GEMV)
    assert ei.value.status == q.QMOE_EUNSUPPORTED
    R = c.T * c.k
    off = torch.zeros((c.E + 1,), dtype=torch.int32, device="cuda")
    p2e = torch.zeros((R,), dtype=torch.int32, device="cuda")
    h = torch.empty((R, c.I), dtype=torch.bfloat16, device="cuda")
    ws = q.alloc_workspace(1 << 20)
    with pytest.raises(q.QmoeError) as ei:          # refused on the host, nothing launched
        q.qmoe_fp4_gemv_fc1_swiglu(bf16_dev(L65.x), c.k, w1, off, p2e, h, ws, path=q.QMOE_PATH_GEMV)
    assert ei.value.status == q.QMOE_EUNSUPPORTED
    check_layer(L65)                                     # 65 rows: AUTO takes the grouped GEMM


# Grouped (prefill) path: several 64-row tiles per hot expert, 16-row sub-tiles,
# both codecs, and the same small shape through both paths.
GROUPED = [
    synth.shrink(synth.MX_PREFILL, E=16, T=64, k=4, H=512, I=256, seed=21),   # 256 rows, Zipf: tiles of 64+
    synth.shrink(synth.MX_PREFILL, E=64, T=128, k=8, H=256, I=128, seed=22),  # 1024 rows
    synth.shrink(synth.DECODE, E=8, T=40, k=2, H=256, I=128, seed=23),        # NVFP4, 80 rows
    synth.shrink(synth.MTP8, E=24, T=24, k=8, H=384, I=192, seed=24),         # NVFP4, hot experts m=24
]


@pytest.mark.parametrize("cfg", GROUPED, ids=lambda c: c.name)
def test_grouped_small(cfg):
    check_layer(synth.layer_inputs(cfg))


@pytest.mark.parametrize("cfg", [synth.shrink(synth.MTP8, E=32, T=8, k=8, H=512, I=256, seed=25),
                                 synth.shrink(synth.MX_DECODE, E=32, T=8, k=8, H=512, I=256, seed=26)],
                         ids=lambda c: c.name)
def test_same_shape_both_paths(cfg):
    import fp4_weight_only_amd as q
    L = synth.layer_inputs(cfg)
    g1 = check_layer(L, path=q.QMOE_PATH_GEMV)
    g2 = check_layer(L, path=q.QMOE_PATH_GROUPED)
    assert np.array_equal(g1["idx"], g2["idx"])
    assert_close("gemv vs grouped", g2["out"], g1["out"])


def test_prefill_full_sampled():
    """4096 routed rows, E=256, hidden 4096, intermediate 2048, MXFP4, Zipf routing."""
    L = synth.layer_inputs(synth.MX_PREFILL)
    rng = np.random.default_rng(1)
    cols1 = np.sort(rng.choice(L.cfg.I, 96, replace=False))
    cols2 = np.sort(rng.choice(L.cfg.H, 128, replace=False))
    check_layer(L, cols1=cols1, cols2=cols2)


POISON_CFGS = [
    synth.shrink(synth.MTP8, E=48, T=8, k=8, H=512, I=384, seed=13),      # hot experts, 64 rows
    synth.shrink(synth.DECODE, E=37, T=7, k=5, H=320, I=144, seed=14),    # ragged K/N, most experts empty
    synth.shrink(synth.MTP4, E=256, T=3, k=8, H=512, I=192, seed=15),     # E = 256: 232+ zero-count experts
]


def _poison_patterns(n_random=24):
    """Float patterns (NaN, +-inf, +-1e30, +-0, float max) and random byte
    patterns, as 32-bit words."""
    vals = np.array([np.nan, np.inf, -np.inf, 1e30, -1e30, 0.0, -0.0, 3.4e38], np.float32).view(np.uint32)
    rng = np.random.default_rng(99)
    return [int(v) for v in vals] + [int(v) for v in rng.integers(0, 2 ** 32, n_random, dtype=np.uint64)]


@pytest.mark.parametrize("cfg", POISON_CFGS, ids=lambda c: c.name)
def test_determinism_and_poisoned_buffers(cfg):
    """Every output and the whole workspace filled with 32 patterns (NaN,
    +-inf, +-1e30, signed zeros, float max, random bytes) before each run: the
    separate calls and the fused calls must reproduce their first results bit
    for bit, on hot, ragged and zero-count expert shapes."""
    L = synth.layer_inputs(cfg)
    layer, logits, x = layer_dev(L)
    print_case("determinism", cfg.name)
    bufs = (layer.topk_idx, layer.topk_w, layer.offsets, layer.p2e, layer.e2p, layer.h, layer.y, layer.out,
            layer.ws)

    def snap():
        return [t.view(torch.uint8).cpu().numpy().copy() for t in bufs[:-1]]

    layer.run(logits, x)
    torch.cuda.synchronize()
    first = snap()
    first_out = bf16_host_from(first[7])

    def fc2_finalize():
        layer.route(logits)
        layer.fc1(x)
        layer.fc2_finalize()

    variants = [("separate", lambda: layer.run(logits, x)), ("fc2+finalize", fc2_finalize)]
    if layer.decode_layer_callable:
        variants.append(("layer decode", lambda: layer.decode_layer(logits, x)))
    if layer.layer_persistent:
        variants.append(("persistent", lambda: layer.persistent_layer(logits, x)))
    for pat in _poison_patterns():
        for name, run in variants:
            for t in bufs:
                fill_pattern(t, pat)
            if layer.ws_layer is not None:   # everything past the counters (they must stay zero)
                fill_pattern(layer.ws_layer[q_layer_sync_bytes():], pat)
            run()
            torch.cuda.synchronize()
            if name == "separate":
                for i, (a, b) in enumerate(zip(first, snap())):
                    assert np.array_equal(a, b), (hex(pat), name, i)
            else:   # h and y are not all written by the fused calls
                assert np.array_equal(bf16_host(layer.out), first_out), (hex(pat), name)
                assert np.array_equal(layer.topk_idx.view(torch.uint8).cpu().numpy(), first[0]), (hex(pat), name)
                if name == "persistent":
                    assert layer_sync_clean(layer.ws_layer), (hex(pat), name)


def bf16_host_from(u8):
    return np.ascontiguousarray(u8).view(np.uint16)


def q_layer_sync_bytes():
    import fp4_weight_only_amd as q
    return q.LAYER_SYNC_BYTES


def layer_sync_clean(ws):
    """The persistent layer's counters are back at zero and its error word is 0."""
    return not bool(ws[:q_layer_sync_bytes()].any().item())


def fill_pattern(t, pat):
    """Fills a device tensor's bytes with the 32-bit word pat repeated."""
    u8 = t.view(torch.uint8).view(-1)
    n = u8.numel()
    rep = np.tile(np.frombuffer(np.uint32(pat).tobytes(), np.uint8), (n + 3) // 4)[:n]
    u8.copy_(torch.from_numpy(np.ascontiguousarray(rep)))


# The same layers against the C++ oracle (plain single-threaded float64,
# written independently of the numpy oracle): the full decode, MTP-verify,
# MXFP4 decode and FP8 layers, a grouped-path batch, the prefill layer on
# sampled columns and the full standalone dequant.
CPP_LAYERS = [synth.TINY, synth.DECODE, synth.MTP4, synth.MTP8, synth.FP8_MTP4, GROUPED[0], GROUPED[3]]


@pytest.mark.parametrize("cfg", CPP_LAYERS, ids=lambda c: c.name)
def test_layer_against_cpp_oracle(cfg):
    check_layer(synth.layer_inputs(cfg), orc="cpp")


@pytest.mark.timeout(600)
def test_layer_mxfp4_decode_full_against_cpp_oracle():
    """The 8-token MXFP4 decode layer (E=256, hidden 4096, intermediate 2048,
    64 rows) on the GEMV path, every column of h, y and out, against the C++
    oracle (about a minute of single-threaded float64 on the host)."""
    check_layer(synth.layer_inputs(synth.MX_DECODE), orc="cpp")


def test_prefill_full_sampled_against_cpp_oracle():
    L = synth.layer_inputs(synth.MX_PREFILL)
    rng = np.random.default_rng(2)
    cols1 = np.sort(rng.choice(L.cfg.I, 48, replace=False))
    cols2 = np.sort(rng.choice(L.cfg.H, 64, replace=False))
    check_layer(L, cols1=cols1, cols2=cols2, orc="cpp")


def test_dequant_full_config_against_cpp_oracle():
    import fp4_weight_only_amd as q
    c = synth.DEQUANT
    w, s, g = synth.dequant_inputs(c)
    out = torch.empty((c.E, c.N, c.K), dtype=torch.bfloat16, device="cuda")
    print_case("dequant full (C++ oracle)", c.name)
    q.qmoe_dequant_fp4(weights_dev(w, s, g, c.fmt), out)
    torch.cuda.synchronize()
    got = bf16_host(out)
    for e in range(c.E):
        assert np.array_equal(got[e], cpp.dequant_bf16(w[e:e + 1], s[e:e + 1], None, c.fmt)[0]), e
