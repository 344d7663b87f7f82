"""Pins for the oracle's absmean ternarization of bf16 weights.

Reading (the pages name absmean quantization and pre-dequantized bf16
checkpoints but give no formula): s = RN32(exact mean |w|), s' = max(s,
1e-5), inv = RN32(1/s'), c = clamp(rne(RN32(w * inv)), -1, 1).

Pins independent of the oracle's code: closed forms (constant magnitudes,
power-of-two means with exact ties), the naive exact-rational sum on small
inputs, numpy's correctly rounded float64 -> float32 conversion for the
final rounding, the exact IEEE model of tests/ieee.py, and invariants.
"""
from fractions import Fraction

import numpy as np
import pytest

from tests import ieee


def bf16(values):
    """float values exactly representable in bf16 -> bit patterns."""
    f = np.asarray(values, np.float32)
    bits = f.view(np.uint32)
    assert np.all(bits & 0xFFFF == 0), "not a bf16 value"
    return (bits >> 16).astype(np.uint16)


def naive_sum(bits):
    out = Fraction(0)
    for b in np.asarray(bits).ravel():
        out += abs(Fraction(float((np.uint32(b) << 16).view(np.float32))))
    return out


def test_rn32_fraction_matches_float64_conversion(oracle_mod):
    # For a value exactly representable in float64, RN32 of it is numpy's
    # correctly rounded float64 -> float32 conversion.
    rng = np.random.default_rng(3)
    vals = np.concatenate([rng.standard_normal(2000) * 10.0 ** rng.integers(-30, 30, 2000),
                           [1 + 2 ** -24, 1 + 3 * 2 ** -25, 2 ** -149 * 1.5, 2 ** -150,
                            3 * 2 ** -151, 1e-40, 0.1, -0.3]])
    for v in vals:
        assert oracle_mod.rn32_fraction(Fraction(float(v))) == np.float32(v), v
    # and agrees with the independent exact model on non-float64 rationals
    for num, den in [(1, 3), (2, 3), (10, 7), (1, 10 ** 9 + 7), (123456789, 1000)]:
        assert Fraction(float(oracle_mod.rn32_fraction(Fraction(num, den)))) == \
            ieee.rn32(Fraction(num, den))


def test_exact_sum_matches_naive(oracle_mod):
    rng = np.random.default_rng(5)
    for shape, scale in [((4, 16), 0.02), ((8, 32), 1.0), ((12, 48), 1e-3)]:
        w = (rng.standard_normal(shape) * scale).astype(np.float32)
        bits = (w.view(np.uint32) >> 16).astype(np.uint16)   # truncate to bf16
        assert oracle_mod.abs_sum_bf16(bits) == naive_sum(bits)
    # extremes: subnormal bf16, the largest finite bf16, zeros of both signs
    bits = np.array([0x0001, 0x8001, 0x007F, 0x0080, 0x7F7F, 0xFF7F, 0x0000, 0x8000],
                    np.uint16)
    assert oracle_mod.abs_sum_bf16(bits) == naive_sum(bits)
    with pytest.raises(oracle_mod.OracleError):
        oracle_mod.abs_sum_bf16(np.array([0x7F80], np.uint16))   # +Inf


def test_constant_magnitude(oracle_mod):
    # |w| = a everywhere: s = a exactly, and every nonzero weight maps to its
    # sign (a * RN32(1/a) rounds to 1).
    for a in (0.01953125, 1.0, 3.0, 2.0 ** -10, 0.0078125):
        w = np.array([[a, -a, a, a], [-a, -a, a, -a]], np.float32)
        codes, s = oracle_mod.ternarize(bf16(w))
        assert s == np.float32(a)
        np.testing.assert_array_equal(codes, np.sign(w).astype(np.int8))


def test_ties_round_half_even(oracle_mod):
    # values {1, 3} in equal numbers: mean 2 exactly, inv = 0.5, so w = 1
    # gives y = 0.5 (tie -> 0) and w = 3 gives 1.5 (-> 2, clamped to 1).
    w = np.array([[1, 3, -1, -3], [3, 1, -3, -1]], np.float32)
    codes, s = oracle_mod.ternarize(bf16(w))
    assert s == np.float32(2.0)
    np.testing.assert_array_equal(codes, [[0, 1, 0, -1], [1, 0, -1, 0]])
    # a zero and values just around the tie: mean of {0, 1.015625, 2.984375,
    # 4} = 2 exactly; 1.015625 * 0.5 = 0.5078125 > 0.5 -> 1
    w = np.array([[0, 1.015625, 2.984375, 4]], np.float32)
    codes, s = oracle_mod.ternarize(bf16(w))
    assert s == np.float32(2.0)
    np.testing.assert_array_equal(codes, [[0, 1, 1, 1]])


def test_mean_rounding_single_step(oracle_mod):
    # mean = 1/3 * (1 + 1 + 2^-7 ...) etc.: the exact quotient rounded once
    rng = np.random.default_rng(9)
    for _ in range(20):
        n = int(rng.integers(1, 64))
        w = bf16(np.round(rng.standard_normal(n) * 64) / 64)
        want = ieee.rn32(naive_sum(w) / n)
        want = max(want, ieee.rn32(Fraction(float(np.float32(1e-5)))))
        assert Fraction(float(oracle_mod.absmean_scale(w))) == want


def test_floor_and_zero(oracle_mod):
    codes, s = oracle_mod.ternarize(np.zeros((4, 16), np.uint16))
    assert s == np.float32(1e-5) and not codes.any()
    # tiny weights: the mean is below the floor, inv = RN32(1/1e-5)
    w = bf16(np.full((4, 16), 2.0 ** -20, np.float32))
    codes, s = oracle_mod.ternarize(w)
    assert s == np.float32(1e-5)
    y = np.float32(2.0 ** -20) * (np.float32(1) / np.float32(1e-5))
    assert np.all(codes == (1 if y > 0.5 else 0))


def test_sign_and_scale_invariance(oracle_mod):
    rng = np.random.default_rng(21)
    w = (rng.standard_normal((8, 64)) * 0.02).astype(np.float32)
    bits = (w.view(np.uint32) >> 16).astype(np.uint16)
    codes, s = oracle_mod.ternarize(bits)
    neg = bits ^ np.uint16(0x8000)
    codes_n, s_n = oracle_mod.ternarize(neg)
    assert s_n == s
    np.testing.assert_array_equal(codes_n, -codes)
    for k in (-3, 5):
        scaled = (((bits.astype(np.uint32) << 16).view(np.float32)) * np.float32(2.0 ** k))
        bk = (scaled.view(np.uint32) >> 16).astype(np.uint16)
        codes_k, s_k = oracle_mod.ternarize(bk)
        assert s_k == np.float32(s * np.float32(2.0 ** k))
        np.testing.assert_array_equal(codes_k, codes)


def test_gaussian_weights_fraction_zero(oracle_mod):
    # For Gaussian weights s -> sigma * E|z| = sigma * sqrt(2/pi), and the rule
    # zeroes |w| < s/2: a fraction P(|z| < sqrt(2/pi)/2) = 0.3108 (N(0, 1)).
    rng = np.random.default_rng(33)
    w = (rng.standard_normal((64, 1024)) * 0.02).astype(np.float32)
    bits = (w.view(np.uint32) >> 16).astype(np.uint16)
    codes, s = oracle_mod.ternarize(bits)
    assert abs(float(s) - 0.02 * np.sqrt(2 / np.pi)) < 0.02 * 0.01
    frac0 = np.mean(codes == 0)
    from math import erf, pi, sqrt
    want = erf(sqrt(2 / pi) / 2 / sqrt(2))
    assert abs(frac0 - want) < 0.01


def tie_matrix():
    """[1920, 4096] weights, all 1.875 except one 0.9375: the exact mean is
    1.875 - 0.9375/7864320 = 1.875 - 2^-23 (an fp32 value), and for the odd
    weight RN32(0.9375 * RN32(1/s)) = 0.5 exactly (code 0), whereas the
    quotient RN32(0.9375 / s) = 0.5 + 2^-24 would give code 1."""
    w = np.full((1920, 4096), 1.875, np.float32)
    w[7, 1000] = 0.9375
    w[::3] *= -1
    return bf16(w)


def test_reciprocal_reading_decides_a_tie(oracle_mod):
    bits = tie_matrix()
    codes, s = oracle_mod.ternarize(bits)
    assert s.view(np.uint32) == 0x3FEFFFFF
    assert Fraction(float(s)) == Fraction(15, 8) - Fraction(1, 2 ** 23)
    inv = np.float32(1) / s
    assert np.float32(np.float32(0.9375) * inv) == np.float32(0.5)
    assert np.float32(np.float32(0.9375) / s) > np.float32(0.5)   # the other reading
    assert codes[7, 1000] == 0
    want = np.where(((bits >> 15) & 1) == 1, -1, 1).astype(np.int8)
    want[7, 1000] = 0
    np.testing.assert_array_equal(codes, want)


def test_exact_sum_not_a_float_accumulation(oracle_mod):
    # 2^24 followed by 255 ones: a running fp32 sum never moves off 2^24,
    # the exact mean is 65536 + 255/256 (an fp32 value).
    w = bf16(np.array([2.0 ** 24] + [1.0] * 255, np.float32))
    assert oracle_mod.absmean_scale(w) == np.float32(65536 + 255 / 256)
    acc = np.float32(0)
    for v in (w.astype(np.uint32) << 16).view(np.float32):
        acc = np.float32(acc + v)
    assert acc / np.float32(256) != np.float32(65536 + 255 / 256)
