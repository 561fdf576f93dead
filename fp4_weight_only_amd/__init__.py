"""Python binding of libqmoe, the gfx950 FP4 weight-only MoE expert path.

Argument marshalling only: every step runs in the HIP kernels of libqmoe.so
(built in-tree by fp4_weight_only_amd.build).  PyTorch supplies device memory
and the current stream; tensors are passed by data_ptr().  Importing this
package raises ImportError when the library is not built: there is no CPU
fallback.

The functions carry the names of the C entry points declared in
include/qmoe.h and raise QmoeError on any status other than QMOE_OK.
"""
from __future__ import annotations

import ctypes
import dataclasses
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libqmoe.so")

QMOE_OK, QMOE_EINVAL, QMOE_EUNSUPPORTED, QMOE_EALIGN, QMOE_EWORKSPACE, QMOE_ELAUNCH = range(6)
QMOE_FMT_NVFP4, QMOE_FMT_MXFP4 = 0, 1
QMOE_PATH_AUTO, QMOE_PATH_GEMV, QMOE_PATH_GROUPED = 0, 1, 2
GEMV_MAX_ROWS = 64

EXPORTS = ("qmoe_route_topk", "qmoe_route_topk_router_weights", "qmoe_fp4_resolve_path", "qmoe_fp4_gemv_fc1_swiglu",
           "qmoe_fp4_route_fc1_swiglu", "qmoe_fp4_moe_layer_decode", "qmoe_fp4_moe_layer_persistent",
           "qmoe_fp4_moe_layer_decode_noalloc",
           "qmoe_fp4_gemv_fc2",
           "qmoe_fp4_gemv_fc2_finalize",
           "qmoe_finalize",
           "qmoe_dequant_fp4", "qmoe_fp8_gemv_fc1_swiglu", "qmoe_fp8_gemv_fc2", "qmoe_dequant_fp8",
           "qmoe_status_str")


class QmoeError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn}: {lib.qmoe_status_str(status).decode()}")


class Fp8WeightsC(ctypes.Structure):
    _fields_ = [("w", ctypes.c_void_p), ("gscale", ctypes.c_void_p),
                ("E", ctypes.c_int32), ("K", ctypes.c_int32), ("N", ctypes.c_int32)]


class Fp4WeightsC(ctypes.Structure):
    _fields_ = [("w", ctypes.c_void_p), ("scales", ctypes.c_void_p), ("gscale", ctypes.c_void_p),
                ("E", ctypes.c_int32), ("K", ctypes.c_int32), ("N", ctypes.c_int32), ("fmt", ctypes.c_int32)]


QMOE_SWIGLU_INTERLEAVED = 1
QMOE_SWIGLU_CONCAT = 2


class SwigluC(ctypes.Structure):
    _fields_ = [("alpha", ctypes.c_float), ("beta", ctypes.c_float), ("limit", ctypes.c_float),
                ("fusion", ctypes.c_int32)]


def _swiglu(act):
    """act: None, (alpha, beta, limit) or (alpha, beta, limit, fusion) -> ctypes pointer or None."""
    if act is None:
        return None
    a = tuple(act)
    return ctypes.byref(SwigluC(*a) if len(a) == 4 else SwigluC(*a, QMOE_SWIGLU_INTERLEAVED))


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built (run: python -m fp4_weight_only_amd.build)")
    L = ctypes.CDLL(LIB_PATH)
    P, I32, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.POINTER(ctypes.c_size_t)
    W = ctypes.POINTER(Fp4WeightsC)
    W8 = ctypes.POINTER(Fp8WeightsC)
    sig = {
        "qmoe_route_topk": [P, I32, I32, I32, P, P, P, P, P, P],
        "qmoe_route_topk_router_weights": [P, P, I32, I32, I32, P, P, P, P, P, P],
        "qmoe_fp4_gemv_fc1_swiglu": [P, I32, I32, W, P, P, ctypes.POINTER(SwigluC), P, P, SZ, I32, P],
        "qmoe_fp4_resolve_path": [I32, I32, W, I32, ctypes.POINTER(ctypes.c_int)],
        "qmoe_fp4_moe_layer_decode": [P, P, P, I32, I32, W, W, ctypes.POINTER(SwigluC), I32, P, P, P, P, P, P, P,
                                      SZ, P],
        "qmoe_fp4_moe_layer_persistent": [P, P, P, I32, I32, W, W, ctypes.POINTER(SwigluC), P, P, P, P, P, P, P,
                                          SZ, P],
        "qmoe_fp4_moe_layer_decode_noalloc": [P, P, P, I32, I32, W, W, ctypes.POINTER(SwigluC), I32, P, P, P, P,
                                              P, P, P],
        "qmoe_fp4_route_fc1_swiglu": [P, P, P, I32, I32, W, ctypes.POINTER(SwigluC), P, P, P, P, P, P, P, SZ, P],
        "qmoe_fp4_gemv_fc2": [P, I32, I32, W, P, P, P, SZ, I32, P],
        "qmoe_fp4_gemv_fc2_finalize": [P, I32, I32, W, P, P, P, P, P, SZ, I32, P],
        "qmoe_finalize": [P, P, P, I32, I32, I32, P, P],
        "qmoe_dequant_fp4": [W, P, P],
        "qmoe_fp8_gemv_fc1_swiglu": [P, I32, I32, W8, P, P, ctypes.POINTER(SwigluC), P, P, SZ, I32, P],
        "qmoe_fp8_gemv_fc2": [P, I32, I32, W8, P, P, P, SZ, I32, P],
        "qmoe_dequant_fp8": [W8, P, P],
    }
    for name, args in sig.items():
        f = getattr(L, name)
        f.argtypes = args
        f.restype = ctypes.c_int
    L.qmoe_status_str.argtypes = [ctypes.c_int]
    L.qmoe_status_str.restype = ctypes.c_char_p
    return L


lib = _load()


@dataclasses.dataclass
class FP4Weights:
    """Device tensors of one FC layer: w [E][K][N/2] uint8, scales [E][K/B][N] uint8, gscale [E] f32 or None."""
    w: torch.Tensor
    scales: torch.Tensor
    gscale: torch.Tensor | None
    fmt: int

    def c(self) -> Fp4WeightsC:
        E, K, half = self.w.shape
        return Fp4WeightsC(self.w.data_ptr(), self.scales.data_ptr(),
                           None if self.gscale is None else self.gscale.data_ptr(), E, K, 2 * half, self.fmt)


@dataclasses.dataclass
class FP8Weights:
    """Device tensors of one FP8 (W8A16) FC layer: w [E][N][K] uint8 E4M3 bytes, gscale [E] f32."""
    w: torch.Tensor
    gscale: torch.Tensor

    def c(self) -> Fp8WeightsC:
        E, N, K = self.w.shape
        return Fp8WeightsC(self.w.data_ptr(), self.gscale.data_ptr(), E, K, N)


def _stream(stream):
    if stream is not None:
        return stream
    return torch.cuda.current_stream().cuda_stream


def _ptr(t):
    return None if t is None else t.data_ptr()


def _check(fn, st):
    if st != QMOE_OK:
        raise QmoeError(fn, st)


def qmoe_route_topk(logits, k, topk_idx, topk_w, expert_offsets, perm_to_expanded, expanded_to_perm, stream=None):
    T, E = logits.shape
    _check("qmoe_route_topk", lib.qmoe_route_topk(
        _ptr(logits), T, E, k, _ptr(topk_idx), _ptr(topk_w), _ptr(expert_offsets), _ptr(perm_to_expanded),
        _ptr(expanded_to_perm), _stream(stream)))


def qmoe_route_topk_router_weights(logits, router_weights, k, topk_idx, topk_w, expert_offsets, perm_to_expanded,
                                   expanded_to_perm, stream=None):
    T, E = logits.shape
    _check("qmoe_route_topk_router_weights", lib.qmoe_route_topk_router_weights(
        _ptr(logits), _ptr(router_weights), T, E, k, _ptr(topk_idx), _ptr(topk_w), _ptr(expert_offsets),
        _ptr(perm_to_expanded), _ptr(expanded_to_perm), _stream(stream)))


def fc_workspace_bytes(which: int, T: int, k: int, w: FP4Weights, path=QMOE_PATH_AUTO, act=None) -> int:
    """Workspace size of qmoe_fp4_gemv_fc1_swiglu (which=1, with its act), qmoe_fp4_gemv_fc2
    (which=2), qmoe_fp4_gemv_fc2_finalize (which=3) or qmoe_fp4_route_fc1_swiglu (which=4,
    with its act; path is ignored)."""
    n = ctypes.c_size_t(0)
    wc = w.c()
    dummy = 256  # aligned non-null placeholders: a size query launches nothing
    if which == 1:
        st = lib.qmoe_fp4_gemv_fc1_swiglu(dummy, T, k, ctypes.byref(wc), dummy, dummy, _swiglu(act), dummy, None,
                                          ctypes.byref(n), path, None)
    elif which == 2:
        st = lib.qmoe_fp4_gemv_fc2(dummy, T, k, ctypes.byref(wc), dummy, dummy, None, ctypes.byref(n), path, None)
    elif which == 4:
        st = lib.qmoe_fp4_route_fc1_swiglu(dummy, None, dummy, T, k, ctypes.byref(wc), _swiglu(act), dummy, dummy,
                                           dummy, dummy, dummy, dummy, None, ctypes.byref(n), None)
    else:
        st = lib.qmoe_fp4_gemv_fc2_finalize(dummy, T, k, ctypes.byref(wc), dummy, dummy, dummy, dummy, None,
                                            ctypes.byref(n), path, None)
    _check("fc_workspace_bytes", st)
    return n.value


def qmoe_fp4_resolve_path(T: int, k: int, w: FP4Weights, path=QMOE_PATH_AUTO) -> int:
    """The path (QMOE_PATH_GEMV or QMOE_PATH_GROUPED) an FC call with these arguments takes."""
    out = ctypes.c_int(-1)
    wc = w.c()
    _check("qmoe_fp4_resolve_path", lib.qmoe_fp4_resolve_path(T, k, ctypes.byref(wc), path, ctypes.byref(out)))
    return out.value


def layer_decode_workspace_bytes(T: int, k: int, w1: FP4Weights, w2: FP4Weights, act=None) -> int:
    """Workspace size of qmoe_fp4_moe_layer_decode."""
    n = ctypes.c_size_t(0)
    c1, c2 = w1.c(), w2.c()
    d = 256
    _check("layer_decode_workspace_bytes", lib.qmoe_fp4_moe_layer_decode(
        d, None, d, T, k, ctypes.byref(c1), ctypes.byref(c2), _swiglu(act), 0, d, d, d, d, d, d, None,
        ctypes.byref(n), None))
    return n.value


def alloc_workspace(nbytes: int, device="cuda") -> torch.Tensor:
    """Workspace of at least nbytes (scratch: its contents do not matter)."""
    return torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)


def qmoe_fp4_gemv_fc1_swiglu(x, k, w1: FP4Weights, expert_offsets, perm_to_expanded, h, ws, act=None,
                             path=QMOE_PATH_AUTO, stream=None):
    T = x.shape[0]
    wc = w1.c()
    n = ctypes.c_size_t(ws.numel() * ws.element_size())
    a = _swiglu(act)
    _check("qmoe_fp4_gemv_fc1_swiglu", lib.qmoe_fp4_gemv_fc1_swiglu(
        _ptr(x), T, k, ctypes.byref(wc), _ptr(expert_offsets), _ptr(perm_to_expanded), a, _ptr(h), _ptr(ws),
        ctypes.byref(n), path, _stream(stream)))


def qmoe_fp4_route_fc1_swiglu(logits, router_weights, x, k, w1: FP4Weights, topk_idx, topk_w, expert_offsets,
                              perm_to_expanded, expanded_to_perm, h, ws, act=None, stream=None):
    T = x.shape[0]
    wc = w1.c()
    n = ctypes.c_size_t(ws.numel() * ws.element_size())
    _check("qmoe_fp4_route_fc1_swiglu", lib.qmoe_fp4_route_fc1_swiglu(
        _ptr(logits), _ptr(router_weights), _ptr(x), T, k, ctypes.byref(wc), _swiglu(act), _ptr(topk_idx),
        _ptr(topk_w), _ptr(expert_offsets), _ptr(perm_to_expanded), _ptr(expanded_to_perm), _ptr(h), _ptr(ws),
        ctypes.byref(n), _stream(stream)))


def qmoe_fp4_moe_layer_decode(logits, router_weights, x, k, w1: FP4Weights, w2: FP4Weights, topk_idx, topk_w,
                              expert_offsets, perm_to_expanded, expanded_to_perm, out, ws, act=None,
                              route_in_fc1=False, stream=None):
    T = x.shape[0]
    c1, c2 = w1.c(), w2.c()
    n = ctypes.c_size_t(ws.numel() * ws.element_size())
    _check("qmoe_fp4_moe_layer_decode", lib.qmoe_fp4_moe_layer_decode(
        _ptr(logits), _ptr(router_weights), _ptr(x), T, k, ctypes.byref(c1), ctypes.byref(c2), _swiglu(act),
        1 if route_in_fc1 else 0, _ptr(topk_idx), _ptr(topk_w), _ptr(expert_offsets), _ptr(perm_to_expanded),
        _ptr(expanded_to_perm), _ptr(out), _ptr(ws), ctypes.byref(n), _stream(stream)))


LAYER_SYNC_BYTES = 69888   # QMOE_LAYER_SYNC_BYTES: counters at the start of the persistent layer's workspace


def layer_persistent_workspace_bytes(T: int, k: int, w1: FP4Weights, w2: FP4Weights, act=None) -> int:
    """Workspace size of qmoe_fp4_moe_layer_persistent."""
    n = ctypes.c_size_t(0)
    c1, c2 = w1.c(), w2.c()
    d = 256
    _check("layer_persistent_workspace_bytes", lib.qmoe_fp4_moe_layer_persistent(
        d, None, d, T, k, ctypes.byref(c1), ctypes.byref(c2), _swiglu(act), d, d, d, d, d, d, None,
        ctypes.byref(n), None))
    return n.value


def alloc_layer_workspace(nbytes: int, device="cuda") -> torch.Tensor:
    """Workspace of qmoe_fp4_moe_layer_persistent: zero-filled once here (its counters must start at
    zero; every completed call leaves them zero)."""
    return torch.zeros(max(nbytes, LAYER_SYNC_BYTES), dtype=torch.uint8, device=device)


def layer_error_word(ws: torch.Tensor) -> int:
    """The persistent layer's error word (bytes 0..3 of its workspace): nonzero after a wait ran out."""
    return int(ws[:4].view(torch.int32).item())


def qmoe_fp4_moe_layer_persistent(logits, router_weights, x, k, w1: FP4Weights, w2: FP4Weights, topk_idx, topk_w,
                                  expert_offsets, perm_to_expanded, expanded_to_perm, out, ws, act=None,
                                  stream=None):
    T = x.shape[0]
    c1, c2 = w1.c(), w2.c()
    n = ctypes.c_size_t(ws.numel() * ws.element_size())
    _check("qmoe_fp4_moe_layer_persistent", lib.qmoe_fp4_moe_layer_persistent(
        _ptr(logits), _ptr(router_weights), _ptr(x), T, k, ctypes.byref(c1), ctypes.byref(c2), _swiglu(act),
        _ptr(topk_idx), _ptr(topk_w), _ptr(expert_offsets), _ptr(perm_to_expanded), _ptr(expanded_to_perm),
        _ptr(out), _ptr(ws), ctypes.byref(n), _stream(stream)))


NOALLOC_SCRATCH_BYTES = 32 << 20


def qmoe_fp4_moe_layer_decode_noalloc(logits, router_weights, x, k, w1: FP4Weights, w2: FP4Weights, topk_idx,
                                      topk_w, expert_offsets, perm_to_expanded, expanded_to_perm, out, act=None,
                                      route_in_fc1=False, stream=None):
    """qmoe_fp4_moe_layer_decode with the library's fixed device scratch (no workspace argument)."""
    T = x.shape[0]
    c1, c2 = w1.c(), w2.c()
    _check("qmoe_fp4_moe_layer_decode_noalloc", lib.qmoe_fp4_moe_layer_decode_noalloc(
        _ptr(logits), _ptr(router_weights), _ptr(x), T, k, ctypes.byref(c1), ctypes.byref(c2), _swiglu(act),
        1 if route_in_fc1 else 0, _ptr(topk_idx), _ptr(topk_w), _ptr(expert_offsets), _ptr(perm_to_expanded),
        _ptr(expanded_to_perm), _ptr(out), _stream(stream)))


def qmoe_fp4_gemv_fc2(h, T, k, w2: FP4Weights, expert_offsets, y_rows, ws, path=QMOE_PATH_AUTO, stream=None):
    wc = w2.c()
    n = ctypes.c_size_t(ws.numel() * ws.element_size())
    _check("qmoe_fp4_gemv_fc2", lib.qmoe_fp4_gemv_fc2(
        _ptr(h), T, k, ctypes.byref(wc), _ptr(expert_offsets), _ptr(y_rows), _ptr(ws), ctypes.byref(n), path,
        _stream(stream)))


def qmoe_fp4_gemv_fc2_finalize(h, k, w2: FP4Weights, expert_offsets, topk_w, expanded_to_perm, out, ws,
                               path=QMOE_PATH_AUTO, stream=None):
    T = out.shape[0]
    wc = w2.c()
    n = ctypes.c_size_t(ws.numel() * ws.element_size())
    _check("qmoe_fp4_gemv_fc2_finalize", lib.qmoe_fp4_gemv_fc2_finalize(
        _ptr(h), T, k, ctypes.byref(wc), _ptr(expert_offsets), _ptr(topk_w), _ptr(expanded_to_perm), _ptr(out),
        _ptr(ws), ctypes.byref(n), path, _stream(stream)))


def qmoe_finalize(y_rows, topk_w, expanded_to_perm, out, stream=None):
    T, k = topk_w.shape
    H = out.shape[1]
    _check("qmoe_finalize", lib.qmoe_finalize(_ptr(y_rows), _ptr(topk_w), _ptr(expanded_to_perm), T, k, H,
                                               _ptr(out), _stream(stream)))


def qmoe_dequant_fp4(w: FP4Weights, out, stream=None):
    wc = w.c()
    _check("qmoe_dequant_fp4", lib.qmoe_dequant_fp4(ctypes.byref(wc), _ptr(out), _stream(stream)))


def fp8_workspace_bytes(which: int, T: int, k: int, w: FP8Weights, act=None, path=QMOE_PATH_AUTO) -> int:
    """Workspace size of qmoe_fp8_gemv_fc1_swiglu (which=1, with its act) or qmoe_fp8_gemv_fc2 (which=2)."""
    n = ctypes.c_size_t(0)
    wc = w.c()
    dummy = 256
    if which == 1:
        st = lib.qmoe_fp8_gemv_fc1_swiglu(dummy, T, k, ctypes.byref(wc), dummy, dummy, _swiglu(act), dummy, None,
                                          ctypes.byref(n), path, None)
    else:
        st = lib.qmoe_fp8_gemv_fc2(dummy, T, k, ctypes.byref(wc), dummy, dummy, None, ctypes.byref(n), path, None)
    _check("fp8_workspace_bytes", st)
    return n.value


def qmoe_fp8_gemv_fc1_swiglu(x, k, w1: FP8Weights, expert_offsets, perm_to_expanded, h, ws, act=None,
                             path=QMOE_PATH_AUTO, stream=None):
    T = x.shape[0]
    wc = w1.c()
    n = ctypes.c_size_t(ws.numel() * ws.element_size())
    _check("qmoe_fp8_gemv_fc1_swiglu", lib.qmoe_fp8_gemv_fc1_swiglu(
        _ptr(x), T, k, ctypes.byref(wc), _ptr(expert_offsets), _ptr(perm_to_expanded), _swiglu(act), _ptr(h),
        _ptr(ws), ctypes.byref(n), path, _stream(stream)))


def qmoe_fp8_gemv_fc2(h, T, k, w2: FP8Weights, expert_offsets, y_rows, ws, path=QMOE_PATH_AUTO, stream=None):
    wc = w2.c()
    n = ctypes.c_size_t(ws.numel() * ws.element_size())
    _check("qmoe_fp8_gemv_fc2", lib.qmoe_fp8_gemv_fc2(
        _ptr(h), T, k, ctypes.byref(wc), _ptr(expert_offsets), _ptr(y_rows), _ptr(ws), ctypes.byref(n), path,
        _stream(stream)))


def qmoe_dequant_fp8(w: FP8Weights, out, stream=None):
    wc = w.c()
    _check("qmoe_dequant_fp8", lib.qmoe_dequant_fp8(ctypes.byref(wc), _ptr(out), _stream(stream)))
