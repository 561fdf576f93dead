"""Helpers for the GPU parity tests: upload synth inputs, download results."""
import numpy as np
import torch

import synth


def to_dev(a, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.view(dtype)
    return t.cuda()


def bf16_dev(bits: np.ndarray) -> torch.Tensor:
    return to_dev(bits.view(np.int16), torch.bfloat16)


def bf16_host(t: torch.Tensor) -> np.ndarray:
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def fmt_code(fmt: str) -> int:
    import fp4_weight_only_amd as q
    return q.QMOE_FMT_NVFP4 if fmt == synth.NVFP4 else q.QMOE_FMT_MXFP4


def weights_dev(w, s, g, fmt):
    import fp4_weight_only_amd as q
    if fmt == "fp8":
        return q.FP8Weights(to_dev(w), to_dev(g))
    return q.FP4Weights(to_dev(w), to_dev(s), None if g is None else to_dev(g), fmt_code(fmt))


def layer_dev(L: synth.LayerInputs, path=None, act=None):
    import fp4_weight_only_amd as q
    from fp4_weight_only_amd.layer import MoELayer
    c = L.cfg
    w1 = weights_dev(L.w1, L.s1, L.g1, c.fmt)
    w2 = weights_dev(L.w2, L.s2, L.g2, c.fmt)
    layer = MoELayer(c.T, c.E, c.k, c.H, c.I, w1, w2, q.QMOE_PATH_AUTO if path is None else path, act)
    return layer, to_dev(L.logits), bf16_dev(L.x)


def print_case(*parts):
    print("CASE", *parts, flush=True)
