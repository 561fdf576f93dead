"""FP4 and FP8 weight dequantization (float64).  Test infrastructure only.

Definition (operator documentation section 6.5 and section 13, "Reference
computation"): a weight is its E2M1 value times its block scale times the
per-expert global scale,

    W[e, k, n] = e2m1(code[e, k, n]) * scale(S[e, k // B, n]) * g[e]

with B = 16 and E4M3FN scales for NVFP4 (section 9b), B = 32 and E8M0 scales
for MXFP4; MXFP4 without a global scale uses g = 1 (reading: the MXFP4
workloads give no global scale).  The packed layout is [E][K][N/2] and the
scale layout [E][K/B][N].

FP8 W8A16 (operator documentation sections 6.4 and 10): raw E4M3FN bytes
laid out [E][N][K] (each output column's K weights contiguous), no block
scales, one float32 global scale per expert applied to the product:

    W[e, k, n] = e4m3(byte[e, n, k]) * g[e]

The bf16 output of the standalone dequant ("[CUDA] Coalesce QMoE MXFP4/NVFP4
weight dequantization") is laid out [E][N][K].  Reading of its rounding: the
product code*scale is exact; multiplying by the float32 global scale rounds
once to float32 (RNE), and the float32 result rounds once to bfloat16 (RNE).
"""
from __future__ import annotations

import numpy as np

from . import codecs


def dequant_expert_f64(w_e, s_e, g_e, fmt: str, cols=None) -> np.ndarray:
    """One expert: packed [K][N/2], scales [K/B][N] -> float64 [K][N] (or [K][len(cols)])."""
    B = 16 if fmt == "nvfp4" else 32
    if cols is None:
        codes = codecs.unpack_codes(w_e)                  # [K][N]
        scales = codecs.block_scale_value(s_e, fmt)       # [K/B][N]
    else:                                                 # only the requested columns
        cols = np.asarray(cols)
        codes = codecs.unpack_column(w_e, cols)
        scales = codecs.block_scale_value(np.asarray(s_e)[:, cols], fmt)
    K = codes.shape[0]
    val = codecs.e2m1_value(codes) * np.repeat(scales, B, axis=0)[:K]
    gv = 1.0 if g_e is None else float(np.float32(g_e))
    return val * gv


def dequant_bf16(w, s, g, fmt: str) -> np.ndarray:
    """All experts: -> bfloat16 bits [E][N][K] per the rounding reading above."""
    E = w.shape[0]
    out = []
    for e in range(E):
        B = 16 if fmt == "nvfp4" else 32
        codes = codecs.unpack_codes(w[e])
        exact = codecs.e2m1_value(codes) * np.repeat(codecs.block_scale_value(s[e], fmt), B, axis=0)
        if g is not None:
            exact = exact * float(np.float32(g[e]))       # exact in float64 (<= 30 significant bits)
        f32 = codecs.f32_round(exact)
        out.append(codecs.bf16_from_f32_bits(f32).T)
    return np.ascontiguousarray(np.stack(out))


def dequant_fp8_expert_f64(w_e, g_e, cols=None) -> np.ndarray:
    """One FP8 expert: bytes [N][K] -> float64 [K][N] (or [K][len(cols)])."""
    w_e = np.asarray(w_e)
    if cols is not None:
        w_e = w_e[np.asarray(cols)]
    return codecs.e4m3fn_value(w_e).T * float(np.float32(g_e))


def dequant_fp8_bf16(w, g) -> np.ndarray:
    """All FP8 experts -> bfloat16 bits [E][N][K]: the product e4m3 * g (at
    most 28 significant bits, exact in float64) rounds once to float32 and
    once to bfloat16, as the FP4 dequant's rounding reading."""
    out = []
    for e in range(w.shape[0]):
        exact = codecs.e4m3fn_value(w[e]) * float(np.float32(g[e]))
        out.append(codecs.bf16_from_f32_bits(codecs.f32_round(exact)))
    return np.ascontiguousarray(np.stack(out))


def expert_weights_f64(w_e, s_e, g_e, fmt: str, cols=None) -> np.ndarray:
    """float64 [K][N] weights of one expert in any of the three codecs."""
    if fmt == "fp8":
        return dequant_fp8_expert_f64(w_e, g_e, cols)
    return dequant_expert_f64(w_e, s_e, g_e, fmt, cols)


def fc_n(w, fmt: str) -> int:
    """Output count N of an FC layer's weight tensor."""
    return w.shape[1] if fmt == "fp8" else 2 * w.shape[2]
