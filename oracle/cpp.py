"""ctypes wrapper of the C++ oracle (qmoe_oracle.cpp).  Test infrastructure only.

The C++ oracle is the plain single-threaded double-precision definition of
the path (codecs, dequant, routing, expert maps, FC1+SwiGLU, FC2, finalize,
the whole layer), written independently of the numpy oracle in this package:
the two share no code, and the tests pin each against closed forms, library
routines, brute force and the other.  Like the rest of ``oracle/`` it is
loaded only by the tests, the smoke check and the benchmark's CPU baseline.

The library is compiled with g++ (``build()``, also run on first use when the
shared object is missing or older than its source); ``-ffp-contract=off``
keeps every multiply and add a separately rounded IEEE operation.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "qmoe_oracle.cpp")
LIB = os.path.join(HERE, "libqmoe_oracle.so")
FMT = {"nvfp4": 0, "mxfp4": 1, "fp8": 2}

_lib = None


def build() -> str:
    tmp = f"{LIB}.tmp{os.getpid()}"  # one temporary per process: concurrent builds do not collide
    cmd = ["g++", "-O2", "-std=c++17", "-Wall", "-Wextra", "-Werror", "-ffp-contract=off",
           "-shared", "-fPIC", SRC, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"oracle build failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
            build()
        L = ctypes.CDLL(LIB)
        P = ctypes.c_void_p
        i32, i64, f64 = ctypes.c_int, ctypes.c_int64, ctypes.c_double
        sig = {
            "qo_e2m1": (f64, [i32]), "qo_e4m3fn": (f64, [i32]), "qo_e8m0": (f64, [i32]),
            "qo_bf16_from_f32": (ctypes.c_uint16, [ctypes.c_float]),
            "qo_bf16_from_f64": (ctypes.c_uint16, [f64]),
            "qo_bf16_from_f32_n": (None, [P, i64, P]), "qo_bf16_from_f64_n": (None, [P, i64, P]),
            "qo_dequant_bf16": (None, [P, P, P, i32, i32, i32, i32, P]),
            "qo_expert_weights_f64": (None, [P, P, P, i32, i32, i32, i32, i32, P]),
            "qo_route_topk": (None, [P, i32, i32, i32, P, P]),
            "qo_route_topk_router_weights": (None, [P, P, i32, i32, i32, P, P]),
            "qo_expert_maps": (None, [P, i32, i32, i32, P, P, P]),
            "qo_fc1_swiglu": (None, [P, i32, P, P, P, i32, i32, i32, i32, P, P, f64, f64, f64, i32, P, i32, P, P]),
            "qo_fc2": (None, [P, P, P, P, i32, i32, i32, i32, P, P, i32, P]),
            "qo_finalize": (None, [P, P, P, i32, i32, i32, P]),
            "qo_layer": (None, [P, P, P, i32, i32, i32, i32, i32, i32, P, P, P, P, P, P, f64, f64, f64, i32,
                                P, P, P, P, P, P, P, P]),
        }
        for name, (res, args) in sig.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def _c(a, dtype):
    """Contiguous array of dtype (None passes through) and its address."""
    if a is None:
        return None, None
    arr = np.ascontiguousarray(a, dtype=dtype)
    return arr, arr.ctypes.data


# ------------------------------------------------------------------ codecs --

def e2m1_value(codes) -> np.ndarray:
    c = np.asarray(codes, np.int64)
    return np.array([lib().qo_e2m1(int(v)) for v in c.reshape(-1)], np.float64).reshape(c.shape)


def e4m3fn_value(bytes_) -> np.ndarray:
    b = np.asarray(bytes_, np.int64)
    return np.array([lib().qo_e4m3fn(int(v)) for v in b.reshape(-1)], np.float64).reshape(b.shape)


def e8m0_value(bytes_) -> np.ndarray:
    b = np.asarray(bytes_, np.int64)
    return np.array([lib().qo_e8m0(int(v)) for v in b.reshape(-1)], np.float64).reshape(b.shape)


def bf16_from_f32_bits(a) -> np.ndarray:
    arr, p = _c(a, np.float32)
    out = np.empty(arr.shape, np.uint16)
    lib().qo_bf16_from_f32_n(p, arr.size, out.ctypes.data)
    return out


def bf16_from_f64(a) -> np.ndarray:
    arr, p = _c(a, np.float64)
    out = np.empty(arr.shape, np.uint16)
    lib().qo_bf16_from_f64_n(p, arr.size, out.ctypes.data)
    return out


# ----------------------------------------------------------------- dequant --

def _dims(w, fmt):
    """(E, K, N) of a weight tensor: FP4 [E][K][N/2], FP8 [E][N][K]."""
    if fmt == "fp8":
        return w.shape[0], w.shape[2], w.shape[1]
    return w.shape[0], w.shape[1], 2 * w.shape[2]


def dequant_bf16(w, s, g, fmt: str) -> np.ndarray:
    """All experts -> bf16 bits [E][N][K]."""
    E, K, N = _dims(w, fmt)
    wa, wp = _c(w, np.uint8)
    sa, sp = _c(s, np.uint8)
    ga, gp = _c(g, np.float32)
    out = np.empty((E, N, K), np.uint16)
    lib().qo_dequant_bf16(wp, sp, gp, E, K, N, FMT[fmt], out.ctypes.data)
    return out


def expert_weights_f64(w, s, g, fmt: str, e: int) -> np.ndarray:
    """Dequantized weights of expert e as float64 [K][N]."""
    E, K, N = _dims(w, fmt)
    wa, wp = _c(w, np.uint8)
    sa, sp = _c(s, np.uint8)
    ga, gp = _c(g, np.float32)
    out = np.empty((K, N), np.float64)
    lib().qo_expert_weights_f64(wp, sp, gp, E, K, N, FMT[fmt], int(e), out.ctypes.data)
    return out


# ----------------------------------------------------------------- routing --

def route_topk(logits, k: int):
    lg, lp = _c(logits, np.float32)
    T, E = lg.shape
    idx = np.empty((T, k), np.int32)
    w = np.empty((T, k), np.float64)
    lib().qo_route_topk(lp, T, E, k, idx.ctypes.data, w.ctypes.data)
    return idx, w


def route_topk_router_weights(logits, router_weights, k: int):
    lg, lp = _c(logits, np.float32)
    rw, rp = _c(router_weights, np.float32)
    T, E = lg.shape
    idx = np.empty((T, k), np.int32)
    w = np.empty((T, k), np.float64)
    lib().qo_route_topk_router_weights(lp, rp, T, E, k, idx.ctypes.data, w.ctypes.data)
    return idx, w


def expert_maps(idx, E: int):
    ia, ip = _c(idx, np.int32)
    T, k = ia.shape
    off = np.empty(E + 1, np.int32)
    p2e = np.empty(T * k, np.int32)
    e2p = np.empty(T * k, np.int32)
    lib().qo_expert_maps(ip, T, k, E, off.ctypes.data, p2e.ctypes.data, e2p.ctypes.data)
    return off, p2e, e2p


# ------------------------------------------------------------------ layers --

def fc1_swiglu(x_bits, k: int, w1, s1, g1, fmt: str, offsets, p2e, act=None, cols=None, want_u=True):
    """-> (h bf16 bits [R][I], u float64 [R][2I] or None).  cols: h columns to compute."""
    act = act or {}
    E, H, N = _dims(w1, fmt)
    I = N // 2
    R = int(offsets[E])
    xa, xp = _c(x_bits, np.uint16)
    wa, wp = _c(w1, np.uint8)
    sa, sp = _c(s1, np.uint8)
    ga, gp = _c(g1, np.float32)
    oa, op = _c(offsets, np.int32)
    pa, pp = _c(p2e, np.int32)
    ca, cp = _c(cols, np.int32)
    h = np.empty((R, I), np.uint16)
    u = np.zeros((R, N), np.float64) if want_u else None
    lib().qo_fc1_swiglu(xp, k, wp, sp, gp, E, H, I, FMT[fmt], op, pp, float(act.get("alpha", 1.0)),
                        float(act.get("beta", 0.0)), float(act.get("limit", np.inf)), int(act.get("fusion", 1)),
                        cp, 0 if ca is None else ca.size, h.ctypes.data, None if u is None else u.ctypes.data)
    return h, u


def fc2(h_bits, w2, s2, g2, fmt: str, offsets, cols=None) -> np.ndarray:
    """-> y float64 [R][H] (or [R][len(cols)])."""
    E, I, H = _dims(w2, fmt)
    R = int(offsets[E])
    ha, hp = _c(h_bits, np.uint16)
    wa, wp = _c(w2, np.uint8)
    sa, sp = _c(s2, np.uint8)
    ga, gp = _c(g2, np.float32)
    oa, op = _c(offsets, np.int32)
    ca, cp = _c(cols, np.int32)
    nc = H if ca is None else ca.size
    y = np.empty((R, nc), np.float64)
    lib().qo_fc2(hp, wp, sp, gp, E, I, H, FMT[fmt], op, cp, 0 if ca is None else ca.size, y.ctypes.data)
    return y


def finalize(y, topk_w, e2p, T: int, k: int) -> np.ndarray:
    ya, yp = _c(y, np.float64)
    wa, wp = _c(topk_w, np.float64)
    ea, ep = _c(e2p, np.int32)
    H = ya.shape[1]
    out = np.empty((T, H), np.float64)
    lib().qo_finalize(yp, wp, ep, T, k, H, out.ctypes.data)
    return out


def layer(inp, act=None, router_weights=None) -> dict:
    """The whole path on a synth.LayerInputs, in one C++ call; every intermediate returned."""
    act = act or {}
    c = inp.cfg
    T, E, k, H, I = c.T, c.E, c.k, c.H, c.I
    R = T * k
    arrs = [_c(inp.logits, np.float32), _c(router_weights, np.float32), _c(inp.x, np.uint16),
            _c(inp.w1, np.uint8), _c(inp.s1, np.uint8), _c(inp.g1, np.float32),
            _c(inp.w2, np.uint8), _c(inp.s2, np.uint8), _c(inp.g2, np.float32)]
    o = dict(idx=np.empty((T, k), np.int32), w=np.empty((T, k), np.float64), offsets=np.empty(E + 1, np.int32),
             p2e=np.empty(R, np.int32), e2p=np.empty(R, np.int32), h=np.empty((R, I), np.uint16),
             y=np.empty((R, H), np.float64), out=np.empty((T, H), np.float64))
    p = [a[1] for a in arrs]
    lib().qo_layer(p[0], p[1], p[2], T, E, k, H, I, FMT[c.fmt], p[3], p[4], p[5], p[6], p[7], p[8],
                   float(act.get("alpha", 1.0)), float(act.get("beta", 0.0)), float(act.get("limit", np.inf)),
                   int(act.get("fusion", 1)),
                   *[o[n].ctypes.data for n in ("idx", "w", "offsets", "p2e", "e2p", "h", "y", "out")])
    return o
