"""Codecs of the FP4 weight formats, written from their definitions (float64).

Test infrastructure only (see the package docstring).

* E2M1 ("MoE and QMoE -- CUDA Operator Documentation", section 9b.3): a 4-bit
  float, bit 3 the sign, bits 2..1 the exponent (bias 1), bit 0 the mantissa;
  exponent field 0 is the subnormal 0.5*m.  Eight magnitudes, two codes per
  byte.
* E4M3FN (the NVFP4 block-scale codec, "[CUDA] Coalesce QMoE MXFP4/NVFP4
  weight dequantization", description of the shared template): sign, 4-bit
  exponent (bias 7), 3-bit mantissa, exponent field 0 subnormal, no infinity,
  only S.1111.111 is NaN; the largest finite value is 448.
* E8M0 / UE8M0 (the MXFP4 block-scale codec, operator documentation section
  6.5): an unsigned 8-bit power-of-two exponent with bias 127; 0xFF is NaN.
* bfloat16 round-to-nearest-even from float32 bits and directly from float64.
"""
from __future__ import annotations

import numpy as np


def e2m1_value(code) -> np.ndarray:
    """Value of 4-bit E2M1 codes (int array, 0..15) as float64."""
    c = np.asarray(code, dtype=np.int64)
    sign = (c >> 3) & 1
    exp = (c >> 1) & 3
    man = c & 1
    mag = np.where(exp == 0, 0.5 * man, np.ldexp(1.0 + 0.5 * man, exp - 1))
    return np.where(sign == 1, -mag, mag)


def e4m3fn_value(byte) -> np.ndarray:
    """Value of E4M3FN bytes (uint8 array) as float64."""
    b = np.asarray(byte, dtype=np.int64)
    sign = (b >> 7) & 1
    exp = (b >> 3) & 15
    man = b & 7
    sub = np.ldexp(man / 8.0, -6)
    nor = np.ldexp(1.0 + man / 8.0, exp - 7)
    mag = np.where(exp == 0, sub, nor)
    mag = np.where((exp == 15) & (man == 7), np.nan, mag)
    return np.where(sign == 1, -mag, mag)


def e8m0_value(byte) -> np.ndarray:
    """Value of E8M0 bytes (uint8 array) as float64: 2^(b-127), 0xFF is NaN."""
    b = np.asarray(byte, dtype=np.int64)
    return np.where(b == 255, np.nan, np.ldexp(1.0, b - 127))


def bf16_from_f32_bits(a_f32) -> np.ndarray:
    """float32 -> bfloat16 bits, round to nearest even; NaN stays a quiet NaN."""
    u = np.asarray(a_f32, dtype=np.float32).view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    nan = np.isnan(np.asarray(a_f32, dtype=np.float32))
    out = np.where(nan, (u >> 16) | 0x40, rounded)
    return out.astype(np.uint16)


def bf16_from_f64(a) -> np.ndarray:
    """float64 -> bfloat16 bits with one round-to-nearest-even step.

    bfloat16 keeps 8 significant bits for normal numbers (exponents -126..127)
    and a fixed quantum of 2^-133 below that; values at or above the rounding
    point past the largest finite number become infinity.
    """
    x = np.asarray(a, dtype=np.float64)
    neg = np.signbit(x)
    mag = np.abs(x)
    _, e = np.frexp(mag)                       # mag = f * 2^e, f in [0.5, 1)
    q_exp = np.maximum(e - 8, -133)            # quantum: 8 significant bits, floor 2^-133
    with np.errstate(over="ignore", invalid="ignore"):
        q = np.ldexp(np.rint(np.ldexp(mag, -q_exp)), q_exp)   # np.rint: ties to even
        q = np.where(np.isinf(mag), np.inf, q)
        q32 = q.astype(np.float32)             # exact (or +inf on overflow)
    bits = (q32.view(np.uint32) >> 16).astype(np.uint32)
    bits = np.where(neg, bits | 0x8000, bits)
    bits = np.where(np.isnan(x), 0x7FC0, bits)
    return bits.astype(np.uint16)


def bf16_to_f64(bits) -> np.ndarray:
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def f32_round(a) -> np.ndarray:
    """float64 -> float32, round to nearest even (IEEE conversion)."""
    with np.errstate(over="ignore"):
        return np.asarray(a, dtype=np.float64).astype(np.float32)


def block_scale_value(byte, fmt: str) -> np.ndarray:
    if fmt == "nvfp4":
        return e4m3fn_value(byte)
    if fmt == "mxfp4":
        return e8m0_value(byte)
    raise ValueError(fmt)


def unpack_codes(packed) -> np.ndarray:
    """[..., N/2] bytes -> [..., N] codes; low nibble is the even column.

    Reading of the packing ("2 per byte along N", operator documentation
    section 6.5; "nibble j of the word is logical element j", PR 31159): the
    low nibble of byte j holds column 2j and the high nibble column 2j+1.
    """
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty(p.shape[:-1] + (p.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = p & 0x0F
    out[..., 1::2] = p >> 4
    return out


def unpack_column(packed, cols) -> np.ndarray:
    """Codes of the given columns n of a [..., N/2] packed array (byte n // 2, nibble n % 2)."""
    p = np.asarray(packed, dtype=np.uint8)
    cols = np.asarray(cols)
    byte = p[..., cols // 2]
    return np.where(cols % 2 == 1, byte >> 4, byte & 0x0F).astype(np.uint8)
