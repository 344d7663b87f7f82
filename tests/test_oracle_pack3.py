"""Pins of the oracle's five-weights-per-byte packing (the denser variant:
the page "Feature request: BitNet 1.58-bit ternary inference on ROCm
(gfx1151)", section "Context", names the TQ1_0 family only, so the layout is
this build's reading; see the fixture for it).

Checked against a hand-derived fixture, exhaustively over all 3^5 columns,
against an independent digit model in Python, with padding rows, reserved
bytes, the packed shapes of the 2B-4T projections, and the product over the
unpacked weights.  The byte form q = ceil(256 v / 243) is chosen so that,
read as the fraction q/256 ~ v/243, the digits come out most significant
first: digit 4 - j is the top of 3 * (q * 3^j mod 256) / 256, a property the
GPU decode uses; it is verified here for every valid byte.
"""
import itertools
import json
import os

import numpy as np
import pytest

import oracle
import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "pack3_example.json")


def test_golden_example():
    g = json.load(open(GOLDEN))
    w = np.array(g["w"], np.int8)
    packed = oracle.pack3(w)
    assert packed.tolist() == g["packed"]
    assert np.array_equal(oracle.unpack3(packed, g["N"]), w)
    for val, q in g["extremes"].items():
        col = np.full((5, 1), int(val), np.int8)
        assert int(oracle.pack3(col)[0, 0]) == q


def digits_model(q):
    """Independent model: v from q by exact rational arithmetic, then base-3."""
    from fractions import Fraction
    v = int(Fraction(243 * q, 256))          # floor(243 q / 256)
    out = []
    for _ in range(5):
        out.append(v % 3)
        v //= 3
    return out


def test_exhaustive_columns():
    cols = np.array(list(itertools.product((-1, 0, 1), repeat=5)), np.int8).T  # [5, 243]
    packed = oracle.pack3(cols)
    assert packed.shape == (1, 243)
    assert len(set(packed[0].tolist())) == 243              # one byte per column
    assert np.array_equal(oracle.unpack3(packed, 5), cols)
    for c in range(243):
        assert digits_model(int(packed[0, c])) == [int(x) + 1 for x in cols[:, c]]


def test_reserved_bytes_rejected():
    cols = np.array(list(itertools.product((-1, 0, 1), repeat=5)), np.int8).T
    valid = set(oracle.pack3(cols)[0].tolist())
    reserved = [b for b in range(256) if b not in valid]
    assert len(reserved) == 13
    for b in reserved:
        with pytest.raises(oracle.OracleError):
            oracle.unpack3(np.array([[b]], np.uint8), 5)


def test_decode_rule_of_the_byte_form():
    # digit 4 - j of v equals (3 * ((q * 3^j) mod 256)) >> 8 for every valid q
    cols = np.array(list(itertools.product((-1, 0, 1), repeat=5)), np.int8).T
    for c, q in enumerate(oracle.pack3(cols)[0].tolist()):
        got = [(3 * ((q * 3 ** j) % 256)) >> 8 for j in range(5)]
        assert got == [int(x) + 1 for x in cols[::-1, c]], q


@pytest.mark.parametrize("N,K", [(1, 16), (4, 32), (7, 48), (11, 64), (640, 96), (2563, 32)])
def test_round_trip_with_padding(N, K):
    w = workloads.ternary_codes(N, K, seed=N + K)
    packed = oracle.pack3(w)
    assert packed.shape == ((N + 4) // 5, K)
    assert np.array_equal(oracle.unpack3(packed, N), w)
    if N % 5:
        # the same bytes read as a taller matrix would need nonzero padding
        # rows to be zero: a nonzero padding digit is rejected
        bad = packed.copy()
        n5 = (N + 4) // 5
        j = N // n5 if N // n5 < 5 else 4
        i = N - j * n5 if N - j * n5 < n5 else n5 - 1
        if j * n5 + i >= N:
            v = (int(bad[i, 0]) * 243) >> 8
            d = (v // 3 ** j) % 3
            v2 = v + (1 if d < 2 else -1) * 3 ** j      # change the padding digit
            bad[i, 0] = (v2 * 256 + 242) // 243
            with pytest.raises(oracle.OracleError):
                oracle.unpack3(bad, N)


def test_shapes_2b4t():
    # five weights per byte: 1.6 bits per weight (plus row padding)
    for N, n5 in [(2560, 512), (640, 128), (6912, 1383), (8192, 1639), (28672, 5735)]:
        assert (N + 4) // 5 == n5


def test_product_over_unpacked_weights():
    N, K = 37, 80
    w = workloads.ternary_codes(N, K, seed=3)
    q = np.random.default_rng(4).integers(-127, 128, (2, K)).astype(np.int8)
    unpacked = oracle.unpack3(oracle.pack3(w), N)
    want = q.astype(np.int64) @ w.astype(np.int64).T
    got = oracle.ternary_matmul(oracle.pack(np.vstack([unpacked, np.zeros((3, K), np.int8)])), q, N + 3)
    assert np.array_equal(got[:, :N], want)


def test_bad_values_rejected():
    with pytest.raises(oracle.OracleError):
        oracle.pack3(np.full((5, 4), 2, np.int8))
