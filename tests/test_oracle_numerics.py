"""Pins of oracle/numerics.py against the pages and a brute-force search."""
import json
import os

import numpy as np
import pytest

from oracle.numerics import (bf16_bits, bf16_rne, f32_bits, f32_from_bits, is_bf16,
                             split_hi_lo)

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _nearest_bf16_bruteforce(x: float) -> float:
    """Nearest BF16 value by comparing the two BF16 neighbours of x in float64;
    an exact halfway case goes to the neighbour whose last fraction bit is 0."""
    if x == 0 or not np.isfinite(x):
        return x
    bits = int(np.array([x], np.float32).view(np.uint32)[0])
    lo_bits = bits & 0xFFFF0000                     # neighbour towards zero
    hi_bits = lo_bits + 0x10000                     # next BF16 away from zero
    lo = float(np.array([lo_bits], np.uint32).view(np.float32)[0])
    hi = float(np.array([hi_bits & 0xFFFFFFFF], np.uint32).view(np.float32)[0])
    dlo, dhi = abs(x - lo), abs(hi - x)
    if dlo < dhi:
        return lo
    if dhi < dlo:
        return hi
    return lo if ((lo_bits >> 16) & 1) == 0 else hi


def test_worked_example_from_the_pages():
    g = json.load(open(os.path.join(GOLD, "bf16_worked_example.json")))
    a = f32_from_bits([int(g["a_bits_fp32"], 2)])[0]
    b = f32_from_bits([int(g["b_bits_fp32"], 2)])[0]
    assert float(a) == g["a_value"] and float(b) == g["b_value"]
    s = np.float32(a) + np.float32(b)                 # FP32 accumulation
    assert format(int(f32_bits([s])[0]), "032b") == g["sum_bits_fp32"]
    assert float(s) == g["sum_value"]
    r = bf16_rne([s])
    assert format(int(bf16_bits(r)[0]), "016b") == g["bf16_bits"]
    assert float(r[0]) == g["bf16_value"]
    assert float(r[0]) - float(s) == g["error"]


def test_bf16_rne_matches_bruteforce_nearest():
    rng = np.random.default_rng(7)
    raw = rng.integers(0, 2**32, size=20000, dtype=np.uint64).astype(np.uint32)
    x = raw.view(np.float32)
    x = x[np.isfinite(x)]
    # halfway cases and their neighbours
    base = rng.integers(0, 2**31, size=2000, dtype=np.uint64).astype(np.uint32) & np.uint32(0x7F7F0000)
    half = (base | np.uint32(0x8000)).view(np.float32)
    near = np.concatenate([half, (base | np.uint32(0x8001)).view(np.float32),
                           (base | np.uint32(0x7FFF)).view(np.float32)])
    x = np.concatenate([x, near, -near, np.float32([1.0, -1.0, 3.0e38, 1e-40])])
    got = bf16_rne(x)
    for xi, gi in zip(x.tolist(), got.tolist()):
        want = _nearest_bf16_bruteforce(xi)
        if np.isfinite(want):
            assert gi == want, (xi, gi, want)
    assert np.all(is_bf16(got[np.isfinite(got)]))


def test_bf16_rne_specials():
    x = np.float32([np.nan, np.inf, -np.inf, 0.0, -0.0])
    r = bf16_rne(x)
    assert np.isnan(r[0]) and r[1] == np.inf and r[2] == -np.inf and r[3] == 0
    assert np.signbit(r[4])
    # the largest finite BF16 plus half an ulp rounds to infinity (ties to even, odd last bit)
    big = f32_from_bits([0x7F7F8000])
    assert bf16_rne(big)[0] == np.inf


def test_split_hi_lo_is_exact_two_term_expansion():
    rng = np.random.default_rng(3)
    p = rng.random(50000).astype(np.float32)
    hi, lo = split_hi_lo(p)
    assert np.all(is_bf16(hi)) and np.all(is_bf16(lo))
    s = hi.astype(np.float64) + lo.astype(np.float64)
    # hi + lo is exactly representable in FP32 and within 2^-16 relative of p
    assert np.all(s.astype(np.float32).astype(np.float64) == s)
    rel = np.abs(s - p) / np.maximum(p, 1e-30)
    assert rel.max() <= 2.0 ** -16


def test_probability_rounds_to_one_window():
    """bf16(exp(-g)) == 1 for gaps up to about 1.955e-3 and < 1 beyond 2.0e-3:
    half a BF16 ulp below 1 is 2^-9."""
    g_in = np.float32([0.0, 1e-4, 1e-3, 1.9e-3])
    g_out = np.float32([2.0e-3, 4e-3])
    assert np.all(bf16_rne(np.exp(-g_in)) == 1.0)
    assert np.all(bf16_rne(np.exp(-g_out)) < 1.0)
    with pytest.raises(AssertionError):
        assert np.all(bf16_rne(np.exp(-np.float32([2.5e-3]))) == 1.0)
