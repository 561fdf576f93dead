"""qmoe_fp4_moe_layer_decode_noalloc (the whole decode layer with the
library's fixed device scratch) against qmoe_fp4_moe_layer_decode (the same
layer with a caller's workspace): every output equal bit for bit, on two calls
in a row whose second input is smaller (the scratch keeps the first call's
contents), and the host-side rejection of shapes the scratch cannot hold."""
import ctypes

import numpy as np
import pytest
import torch

import synth
from gpu_util import layer_dev, print_case, to_dev

pytestmark = pytest.mark.gpu

GPTOSS_CONCAT = (1.702, 1.0, 7.0, 2)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import fp4_weight_only_amd  # noqa: F401  (raises if the library is not built)


def _outputs(layer):
    return (layer.topk_idx, layer.topk_w, layer.offsets, layer.p2e, layer.e2p, layer.out)


def _host(ts):
    return [t.view(torch.int32 if t.element_size() == 4 else torch.int16).cpu().numpy().copy() for t in ts]


def _run_pair(cfg, act=None, rw_on=False, route_in_fc1=False):
    import fp4_weight_only_amd as q
    L = synth.layer_inputs(cfg)
    layer, logits, x = layer_dev(L, act=act, path=q.QMOE_PATH_GEMV)
    rw = to_dev(synth.router_weights(cfg)) if rw_on else None
    print_case("noalloc", cfg.name, "act", act, "router_weights", rw_on, "route_in_fc1", route_in_fc1)
    layer.decode_layer(logits, x, rw, route_in_fc1=route_in_fc1)
    torch.cuda.synchronize()
    ref = _host(_outputs(layer))
    for t in _outputs(layer):                       # poison every output
        t.view(torch.int32 if t.element_size() == 4 else torch.int16).fill_(-7)
    q.qmoe_fp4_moe_layer_decode_noalloc(logits, rw, x, cfg.k, layer.w1, layer.w2, layer.topk_idx, layer.topk_w,
                                        layer.offsets, layer.p2e, layer.e2p, layer.out, act=act,
                                        route_in_fc1=route_in_fc1)
    torch.cuda.synchronize()
    for name, got, r in zip(("idx", "w", "offsets", "p2e", "e2p", "out"), _host(_outputs(layer)), ref):
        assert np.array_equal(got, r), (cfg.name, name)


def test_noalloc_equals_workspace_call_twice_smaller_second():
    # first the 4-token MTP verify layer (32 rows, E = 256, hidden 2048), then
    # a smaller layer (fewer rows, shorter K and N) in the same scratch
    _run_pair(synth.MTP4)
    _run_pair(synth.shrink(synth.DECODE, E=37, T=7, k=5, H=320, I=144, seed=1))


def test_noalloc_variants():
    # routing inside FC1, router weights, GPT-OSS concatenated SwiGLU, MXFP4
    _run_pair(synth.DECODE, route_in_fc1=True)
    _run_pair(synth.shrink(synth.MTP8, E=64, T=8, k=8, H=512, I=272, seed=2), act=GPTOSS_CONCAT, rw_on=True)
    _run_pair(synth.shrink(synth.MX_DECODE, E=12, T=16, k=4, H=1024, I=256, seed=25))
    _run_pair(synth.TINY)


def test_noalloc_rejects_shapes_past_the_scratch():
    """64 rows of a hidden 8192 / intermediate 4096 layer need 67 MB of
    partial sums: refused on the host before any launch."""
    import fp4_weight_only_amd as q
    A = 256   # aligned placeholders: nothing is dereferenced on this path
    w1 = q.Fp4WeightsC(A, A, A, 8, 8192, 8192, q.QMOE_FMT_NVFP4)
    w2 = q.Fp4WeightsC(A, A, A, 8, 4096, 8192, q.QMOE_FMT_NVFP4)
    st = q.lib.qmoe_fp4_moe_layer_decode_noalloc(A, None, A, 8, 8, ctypes.byref(w1), ctypes.byref(w2), None, 0,
                                                 A, A, A, A, A, A, None)
    assert st == q.QMOE_EWORKSPACE
    n = ctypes.c_size_t(0)
    assert q.lib.qmoe_fp4_moe_layer_decode(A, None, A, 8, 8, ctypes.byref(w1), ctypes.byref(w2), None, 0, A, A, A, A,
                                           A, A, None, ctypes.byref(n), None) == q.QMOE_OK
    assert n.value > q.NOALLOC_SCRATCH_BYTES
