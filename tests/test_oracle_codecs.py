"""Pins for the oracle's codecs (CPU only).

Each codec is checked against something other than its own formula: the
golden E2M1 table (OCP MX values), torch's float8_e4m3fn / float8_e8m0fnu
and bfloat16 casts (library routines), and a brute-force nearest-bfloat16
search over all 65536 bit patterns with exact rational arithmetic.
"""
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import codecs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def golden_e2m1():
    vals = {}
    with open(os.path.join(GOLDEN, "e2m1_values.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            c, v = line.split()
            vals[int(c)] = float(v)
    assert len(vals) == 16
    return vals


def test_e2m1_all_codes_match_golden_table():
    g = golden_e2m1()
    got = codecs.e2m1_value(np.arange(16))
    for c in range(16):
        assert got[c] == g[c], c
        assert np.signbit(got[c]) == np.signbit(g[c]), c   # code 8 is -0


def test_e2m1_eight_magnitudes_and_sign_bit():
    v = codecs.e2m1_value(np.arange(16))
    assert sorted(set(np.abs(v).tolist())) == [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    assert np.array_equal(v[8:], -v[:8])


def test_e4m3fn_all_256_bytes_match_torch():
    b = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = b.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = codecs.e4m3fn_value(np.arange(256))
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


def test_e4m3fn_landmarks():
    v = codecs.e4m3fn_value(np.arange(256))
    assert v[0x7E] == 448.0 and np.nanmax(v) == 448.0
    assert np.isnan(v[0x7F]) and np.isnan(v[0xFF]) and np.isnan(v).sum() == 2
    assert v[0x38] == 1.0 and v[0x01] == 2.0 ** -9 and v[0x08] == 2.0 ** -6
    assert np.all(np.diff(v[:0x7F]) > 0)          # monotone in the magnitude bits


def test_e8m0_all_256_bytes_match_torch():
    b = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = b.view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    got = codecs.e8m0_value(np.arange(256))
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan) and nan.sum() == 1 and nan[255]
    assert np.array_equal(got[~nan], ref[~nan])
    assert got[127] == 1.0 and got[0] == 2.0 ** -127


def test_bf16_from_f32_matches_torch():
    rng = np.random.default_rng(7)
    a = np.concatenate([
        rng.standard_normal(20000).astype(np.float32) * np.float32(1e3),
        rng.integers(0, 2 ** 32, 20000, dtype=np.uint64).astype(np.uint32).view(np.float32),
        np.array([0.0, -0.0, np.inf, -np.inf, 3.3895314e38, 1e-45, -1e-40], np.float32),
    ])
    ref = torch.from_numpy(a).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = codecs.bf16_from_f32_bits(a)
    nan = np.isnan(a)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.all((got[nan] & 0x7FC0) == 0x7FC0)


def _bf16_table():
    bits = np.arange(0x7F80, dtype=np.uint32)          # +0 .. largest finite
    vals = (bits << 16).view(np.float32).astype(np.float64)
    return bits, vals


def _nearest_bf16_bruteforce(x: float) -> int:
    """Nearest bfloat16 by search, ties to the even bit pattern (exact rationals)."""
    bits, vals = _bf16_table()
    mag = abs(x)
    i = int(np.searchsorted(vals, mag))
    cands = [j for j in (i - 1, i) if 0 <= j < len(vals)]
    best = None
    for j in cands:
        d = abs(Fraction(mag) - Fraction(float(vals[j])))
        key = (d, int(bits[j]) & 1)
        if best is None or key < best[0]:
            best = (key, int(bits[j]))
    out = best[1]
    if i >= len(vals):                                   # beyond the largest finite value
        top = Fraction(float(vals[-1]))
        half_ulp = Fraction(2) ** (127 - 8)
        if Fraction(mag) >= top + half_ulp:
            out = 0x7F80
    return out | (0x8000 if np.signbit(x) else 0)


def test_bf16_from_f64_single_rounding_bruteforce():
    rng = np.random.default_rng(3)
    xs = list(rng.standard_normal(300) * 10.0 ** rng.integers(-40, 39, 300))
    # ties and near-ties where rounding through float32 first would differ
    one = 1.0
    xs += [one + 2.0 ** -8, one + 3 * 2.0 ** -8, one + 2.0 ** -8 + 2.0 ** -40, one + 2.0 ** -8 - 2.0 ** -40,
           -(one + 2.0 ** -8 + 2.0 ** -40), 2.0 ** -130 * 1.5, 2.0 ** -133 * 0.5, 2.0 ** -133 * 0.75,
           3.3961e38, 3.40e38, 0.0, -0.0]
    for x in xs:
        got = int(codecs.bf16_from_f64(np.array([x]))[0])
        assert got == _nearest_bf16_bruteforce(float(x)), x


def test_bf16_from_f64_agrees_with_torch_on_float32_inputs():
    rng = np.random.default_rng(5)
    a = (rng.standard_normal(50000) * 100).astype(np.float32)
    ref = torch.from_numpy(a).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(codecs.bf16_from_f64(a.astype(np.float64)), ref)


def test_unpack_low_nibble_is_even_column():
    p = np.array([[0x21, 0xF0]], np.uint8)
    assert codecs.unpack_codes(p).tolist() == [[1, 2, 0, 15]]
    assert codecs.unpack_column(p, np.array([3, 0, 1])).tolist() == [[15, 1, 2]]


@pytest.mark.parametrize("b", [0x7F, 0xFF])
def test_e4m3_nan_bytes(b):
    assert np.isnan(codecs.e4m3fn_value(np.array([b])))[0]
