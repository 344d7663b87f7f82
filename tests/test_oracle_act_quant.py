"""Pins for the oracle's per-token absmax int8 activation quantization.

Definition (reading; the pages do not describe activation quantization):
a = max|x|, a' = max(a, 1e-5), inv = RN32(127 / a'),
q = clamp(round_half_even(RN32(x * inv)), -127, 127), s_x = RN32(a' / 127).

Pins are independent of the C code: ties and exact power-of-two scales
(closed forms), an exact-rational model of the IEEE-754 operations
(tests/ieee.py), the quantization error bound, and invariants.
"""
from fractions import Fraction

import numpy as np
import pytest

import workloads
from tests import ieee


def f32(v):
    return np.array(v, np.float32)


def test_ties_round_half_even(oracle_mod):
    # a = 127 makes inv = 127/127 = 1 exactly, so q = rne(x) with no product
    # rounding: ties go to the even neighbour.
    x = f32([[127.0, 0.5, 1.5, 2.5, -2.5, 126.5, -0.5, 3.5, -125.5, 0.49999997]])
    q, s = oracle_mod.act_quant(x, "f32")
    assert q.tolist() == [[127, 0, 2, 2, -2, 126, 0, 4, -126, 0]]
    assert s[0] == np.float32(1.0)


@pytest.mark.parametrize("e", [-12, -3, 0, 5, 20])
def test_exhaustive_bf16_power_of_two_scale(oracle_mod, e):
    # a = 127 * 2^e: inv = 2^-e exactly, so q = rne(x * 2^-e) exactly, for
    # every finite bf16 x with |x| <= a (all 65536 patterns, filtered).
    a = np.float32(127.0 * 2.0 ** e)
    bits = np.arange(1 << 16, dtype=np.uint32)
    xs = (bits << 16).view(np.float32)
    keep = np.isfinite(xs) & (np.abs(xs) <= a)
    xs = xs[keep]
    row = np.concatenate([[a], xs]).astype(np.float32)
    q, s = oracle_mod.act_quant(row[None, :], "f32")
    want = np.rint(row.astype(np.float64) * 2.0 ** (-e))   # exact product
    np.testing.assert_array_equal(q[0].astype(np.float64), want)
    assert s[0] == np.float32(2.0 ** e)


def _model(xs, ap):
    """Exact IEEE model: inv = RN32(127/a'), q = rne(RN32(x inv))."""
    inv = ieee.rn32(Fraction(127) / Fraction(float(ap)))
    out = []
    for x in xs:
        t = ieee.rn32(Fraction(float(x)) * inv)
        out.append(max(-127, min(127, ieee.rne_int(t))))
    return out, ieee.rn32(Fraction(float(ap)) / 127)


def test_ieee_model_random_rows(oracle_mod):
    rng = np.random.default_rng(7)
    for trial in range(40):
        K = int(rng.integers(1, 40))
        scale = float(2.0 ** rng.integers(-20, 20))
        x = (rng.standard_normal(K) * scale).astype(np.float32)
        if trial % 3 == 0:                       # force near-ties
            a = np.max(np.abs(x))
            inv = np.float32(127.0) / np.float32(a)
            x[:-1] = (np.round(x[:-1] * inv) + 0.5).astype(np.float32) / inv
            x = np.clip(x, -a, a).astype(np.float32)
        q, s = oracle_mod.act_quant(x[None, :], "f32")
        ap = max(float(np.max(np.abs(x))), float(np.float32(1e-5)))
        want_q, want_s = _model(x, np.float32(ap))
        assert q[0].tolist() == want_q
        assert Fraction(float(s[0])) == want_s


def test_ieee_model_bf16_sweep(oracle_mod):
    # All finite bf16 values below an absmax of 3.0 (inexact inv = 127/3).
    bits = np.arange(1 << 16, dtype=np.uint32)
    xs = (bits << 16).view(np.float32)
    a = np.float32(3.0)
    keep = np.isfinite(xs) & (np.abs(xs) <= a) & (np.abs(xs) > 0.004)
    row = np.concatenate([[a], xs[keep]]).astype(np.float32)
    q, s = oracle_mod.act_quant(row[None, :], "f32")
    want_q, want_s = _model(row, a)
    assert q[0].tolist() == want_q
    assert Fraction(float(s[0])) == want_s


def test_bf16_entry_matches_widened_f32(oracle_mod):
    xb = workloads.activations_bf16(3, 257, seed=11, outliers=True)
    xf = (xb.astype(np.uint32) << 16).view(np.float32)
    qb, sb = oracle_mod.act_quant(xb, "bf16")
    qf, sf = oracle_mod.act_quant(xf, "f32")
    np.testing.assert_array_equal(qb, qf)
    np.testing.assert_array_equal(sb, sf)
    # The C widening agrees with the bit-level definition (bf16 = top half).
    np.testing.assert_array_equal(oracle_mod.bf16_to_f32(xb[0, :50]), xf[0, :50])


def test_error_bound_and_extremes(oracle_mod):
    x = workloads.normal_f32(8, 2560, seed=3, outliers=True)
    q, s = oracle_mod.act_quant(x, "f32")
    a = np.max(np.abs(x.astype(np.float64)), axis=1, keepdims=True)
    exact = x.astype(np.float64) * 127.0 / a
    # one rounding of inv and one of the product: |err| <= 127 * 2^-23
    assert np.all(np.abs(q - exact) <= 0.5 + 127 * 2.0 ** -22)
    assert q.min() >= -127 and q.max() <= 127
    idx = np.argmax(np.abs(x), axis=1)
    for m in range(8):
        assert abs(int(q[m, idx[m]])) == 127
        assert np.sign(q[m, idx[m]]) == np.sign(x[m, idx[m]])
    # s_x is a'/127 to within one rounding
    assert np.all(np.abs(s.astype(np.float64) - a[:, 0] / 127) <= a[:, 0] / 127 * 2.0 ** -24)


def test_symmetry_and_scale_invariance(oracle_mod):
    x = workloads.normal_f32(4, 300, seed=5)
    q, s = oracle_mod.act_quant(x, "f32")
    qn, sn = oracle_mod.act_quant(-x, "f32")
    np.testing.assert_array_equal(qn, -q)
    np.testing.assert_array_equal(sn, s)
    for e in (-10, -1, 1, 7):
        qe, se = oracle_mod.act_quant((x * np.float32(2.0 ** e)).astype(np.float32), "f32")
        np.testing.assert_array_equal(qe, q)
        np.testing.assert_array_equal(se, (s * np.float32(2.0 ** e)).astype(np.float32))


def test_monotone(oracle_mod):
    x = np.sort(workloads.normal_f32(1, 999, seed=9)[0])
    q, _ = oracle_mod.act_quant(x[None, :], "f32")
    assert np.all(np.diff(q[0].astype(np.int32)) >= 0)


def test_zero_and_tiny_rows(oracle_mod):
    q, s = oracle_mod.act_quant(np.zeros((2, 64), np.float32), "f32")
    assert not q.any()
    assert Fraction(float(s[0])) == ieee.rn32(Fraction(float(np.float32(1e-5))) / 127)
    # 0 < a < 1e-5: the floor a' = 1e-5 applies, nothing saturates.
    x = np.zeros((1, 8), np.float32)
    x[0, 3] = np.float32(5e-6)
    x[0, 5] = np.float32(-2.5e-6)
    q, s = oracle_mod.act_quant(x, "f32")
    want_q, want_s = _model(x[0], np.float32(1e-5))
    assert q[0].tolist() == want_q
    assert abs(int(q[0, 3]) - 63.5) <= 1 and abs(int(q[0, 5]) + 31.75) <= 1
    assert np.abs(q).max() < 127
    # a row of one denormal still gives 0 and a finite scale
    x = np.zeros((1, 4), np.float32)
    x[0, 0] = np.float32(1e-40)
    q, s = oracle_mod.act_quant(x, "f32")
    assert not q.any() and np.isfinite(s).all()


def test_empty(oracle_mod):
    q, s = oracle_mod.act_quant(np.zeros((3, 0), np.float32), "f32")
    assert q.shape == (3, 0)
    assert np.all(s == np.float32(np.float32(1e-5) / np.float32(127.0)))


def test_ieee_helper_known_values():
    # The exact-rational helper itself, against known binary32 facts.
    assert ieee.rn32(Fraction(1, 3)) == Fraction(0x0AAAAAB, 1 << 25)
    one_ulp = Fraction(1, 1 << 23)
    assert ieee.rn32(1 + one_ulp / 2) == 1                   # tie -> even
    assert ieee.rn32(1 + 3 * one_ulp / 2) == 1 + 2 * one_ulp  # tie -> even
    assert ieee.rn32(Fraction(1, 1 << 149)) == Fraction(1, 1 << 149)
    assert ieee.rn32(Fraction(1, 1 << 150)) == 0              # tie -> 0 (even)
    assert ieee.rne_int(Fraction(5, 2)) == 2 and ieee.rne_int(Fraction(-5, 2)) == -2


def _unclamped_peak(a):
    """rne(RN32(a * RN32(127 / max(a, 1e-5)))) in numpy float32: the largest
    unclamped code a row with absmax a can produce (at its absmax element)."""
    a = np.asarray(a, np.float32)
    ap = np.maximum(a, np.float32(1e-5))
    inv = (np.float32(127.0) / ap).astype(np.float32)
    return np.rint((a * inv).astype(np.float32))


def test_clamp_never_binds():
    # The symmetric clamp of the quantization rule is a no-op for finite
    # rows: |x| <= a' and inv = RN32(127/a') give RN32(|x| inv) <= 127 + 2^-17,
    # so |rne(.)| <= 127.  (The GPU kernels rely on this and round without
    # clamping.)  Exhaustive over every positive finite bf16 absmax, and over
    # every fp32 significand in [1, 2) (all exponents scale exactly between
    # 1e-5 and the overflow limit); the product is monotone in |x|, so the
    # absmax element is the worst case of its row.
    bits = np.arange(1, 0x7F80, dtype=np.uint32) << 16
    a_bf16 = bits.view(np.float32)
    peak = _unclamped_peak(a_bf16)
    assert peak.max() == 127.0
    np.testing.assert_array_equal(peak[a_bf16 >= np.float32(1e-5)], 127.0)
    assert np.all(peak[a_bf16 < np.float32(1e-5)] <= 127.0)
    sig = (np.uint32(0x3F800000) + np.arange(1 << 23, dtype=np.uint32)).view(np.float32)
    for e in (-16, 0, 60, 126):
        a = (sig * np.float32(2.0 ** e)).astype(np.float32)
        a = a[np.isfinite(a)]
        np.testing.assert_array_equal(_unclamped_peak(a), 127.0)
    # The same bound from the exact IEEE model (no numpy float32 arithmetic).
    rng = np.random.default_rng(11)
    for a in rng.choice(a_bf16[a_bf16 >= np.float32(1e-5)], 300, replace=False):
        inv = ieee.rn32(Fraction(127) / Fraction(float(a)))
        y = ieee.rn32(Fraction(float(a)) * inv)
        assert y <= 127 + Fraction(1, 1 << 17) and ieee.rne_int(y) == 127
