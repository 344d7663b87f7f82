"""Pins for the oracle's exact ternary product, rescale and relu^2.

The product acc[m,n] = sum_k W[n,k] q[m,k] is checked against brute force in
pure Python, numpy's int64 matmul on the generator's (never packed) codes,
and closed forms.  The rescale and relu^2 are checked against exact rational
models (tests/ieee.py) and their rounding-error bounds.
"""
import itertools
from fractions import Fraction

import numpy as np
import pytest

import workloads
from tests import ieee


def test_bruteforce_all_weights_n4_k2(oracle_mod):
    q = np.array([[3, -5], [-127, 127], [0, 1]], np.int8)
    for ws in itertools.product((-1, 0, 1), repeat=8):
        w = np.array(ws, np.int8).reshape(4, 2)
        acc = oracle_mod.ternary_matmul(oracle_mod.pack(w), q, 4)
        for m in range(3):
            for n in range(4):
                want = 0
                for k in range(2):
                    want += int(w[n, k]) * int(q[m, k])
                assert acc[m, n] == want


@pytest.mark.parametrize("M,N,K", [(1, 8, 8), (2, 4, 7), (3, 8, 5), (1, 4, 1)])
def test_bruteforce_random_tiny(oracle_mod, M, N, K):
    rng = np.random.default_rng(M * 100 + N * 10 + K)
    for _ in range(20):
        w = rng.integers(-1, 2, size=(N, K)).astype(np.int8)
        q = rng.integers(-127, 128, size=(M, K)).astype(np.int8)
        acc = oracle_mod.ternary_matmul(oracle_mod.pack(w), q, N)
        for m in range(M):
            for n in range(N):
                assert acc[m, n] == sum(int(w[n, k]) * int(q[m, k]) for k in range(K))


@pytest.mark.parametrize("M,N,K", [(1, 64, 2560), (5, 132, 1000), (16, 40, 6912)])
def test_numpy_matmul(oracle_mod, M, N, K):
    w = workloads.ternary_codes(N, K, seed=N + K)
    q = np.random.default_rng(K).integers(-127, 128, size=(M, K)).astype(np.int8)
    acc = oracle_mod.ternary_matmul(oracle_mod.pack(w), q, N)
    want = q.astype(np.int64) @ w.astype(np.int64).T
    np.testing.assert_array_equal(acc, want)


def test_rows_subset(oracle_mod):
    N, K = 48, 300
    w = workloads.ternary_codes(N, K, seed=1)
    q = np.random.default_rng(2).integers(-127, 128, size=(3, K)).astype(np.int8)
    p = oracle_mod.pack(w)
    rows = np.array([0, 47, 12, 13, 36, 11])
    sub = oracle_mod.ternary_matmul_rows(p, q, N, rows)
    np.testing.assert_array_equal(sub, oracle_mod.ternary_matmul(p, q, N)[:, rows])


def test_closed_forms(oracle_mod):
    N = K = 64
    q = np.random.default_rng(3).integers(-127, 128, size=(2, K)).astype(np.int8)
    sq = q.astype(np.int64).sum(axis=1)

    def run(w):
        return oracle_mod.ternary_matmul(oracle_mod.pack(w.astype(np.int8)), q, N)

    assert not run(np.zeros((N, K))).any()                         # all-zero
    np.testing.assert_array_equal(run(np.ones((N, K))), np.repeat(sq[:, None], N, 1))
    np.testing.assert_array_equal(run(-np.ones((N, K))), -np.repeat(sq[:, None], N, 1))
    np.testing.assert_array_equal(run(np.eye(N)), q)               # +I
    np.testing.assert_array_equal(run(-np.eye(N)), -q)             # -I
    n_idx, k_idx = np.meshgrid(np.arange(N), np.arange(K), indexing="ij")
    cb = np.where((n_idx + k_idx) % 2 == 0, 1, -1)                 # checkerboard
    alt = (q.astype(np.int64) * np.where(np.arange(K) % 2 == 0, 1, -1)).sum(1)
    want = np.stack([alt[m] * np.where(np.arange(N) % 2 == 0, 1, -1) for m in range(2)])
    np.testing.assert_array_equal(run(cb), want)


def test_one_hot_columns_pin_plane_mapping(oracle_mod):
    # q = 127 e_k reads out column k of W: acc[:, n] = 127 W[n, k].
    N, K = 16, 9
    w = workloads.ternary_codes(N, K, seed=4)
    p = oracle_mod.pack(w)
    for k in range(K):
        q = np.zeros((1, K), np.int8)
        q[0, k] = 127
        np.testing.assert_array_equal(oracle_mod.ternary_matmul(p, q, N)[0], 127 * w[:, k])


def test_invariants(oracle_mod):
    N, K = 24, 200
    w = workloads.ternary_codes(N, K, seed=8)
    p = oracle_mod.pack(w)
    rng = np.random.default_rng(9)
    q1 = rng.integers(-60, 61, size=(1, K)).astype(np.int8)
    q2 = rng.integers(-60, 61, size=(1, K)).astype(np.int8)
    a1 = oracle_mod.ternary_matmul(p, q1, N)
    a2 = oracle_mod.ternary_matmul(p, q2, N)
    np.testing.assert_array_equal(oracle_mod.ternary_matmul(p, q1 + q2, N), a1 + a2)
    perm = rng.permutation(K)
    pp = oracle_mod.pack(w[:, perm])
    np.testing.assert_array_equal(oracle_mod.ternary_matmul(pp, q1[:, perm], N), a1)
    np.testing.assert_array_equal(oracle_mod.ternary_matmul(oracle_mod.pack(-w), q1, N), -a1)


def test_empty_shapes(oracle_mod):
    assert oracle_mod.ternary_matmul(np.zeros((2, 0), np.uint8),
                                     np.zeros((1, 0), np.int8), 8).tolist() == [[0] * 8]
    assert oracle_mod.ternary_matmul(np.zeros((0, 5), np.uint8),
                                     np.zeros((3, 5), np.int8), 0).shape == (3, 0)


def test_int32_range_check(oracle_mod):
    K = (1 << 31) // 127 + 2
    w = np.ones((4, K), np.int8)
    q = np.full((1, K), 127, np.int8)
    with pytest.raises(oracle_mod.OracleError):
        oracle_mod.ternary_matmul(oracle_mod.pack(w), q, 4)


# ---------------------------------------------------------------- rescale
def test_rescale_exact_model(oracle_mod):
    rng = np.random.default_rng(10)
    acc = rng.integers(-127 * 6912, 127 * 6912, size=(3, 50)).astype(np.int32)
    s_x = (np.abs(rng.standard_normal(3)) * 0.05 + 1e-4).astype(np.float32)
    s_w = np.float32(0.023)
    y = oracle_mod.rescale(acc, s_w, s_x)
    y64 = oracle_mod.rescale(acc, s_w, s_x, exact=True)
    for m in range(3):
        c = ieee.rn32(Fraction(float(s_w)) * Fraction(float(s_x[m])))
        for n in range(50):
            want = ieee.rn32(Fraction(int(acc[m, n])) * c)
            assert Fraction(float(y[m, n])) == want
            exact = Fraction(int(acc[m, n])) * Fraction(float(s_w)) * Fraction(float(s_x[m]))
            assert abs(Fraction(float(y64[m, n])) - exact) <= abs(exact) * Fraction(1, 1 << 52)
    rel = np.abs(y - y64) / np.maximum(np.abs(y64), 1e-300)
    assert rel.max() <= 2 * 2.0 ** -24 * (1 + 2.0 ** -23)


def test_rescale_power_of_two_exact(oracle_mod):
    acc = np.array([[0, 1, -1, 127 * 2560, -3]], np.int32)
    y = oracle_mod.rescale(acc, np.float32(2.0 ** -6), np.array([1.0], np.float32))
    np.testing.assert_array_equal(y, acc.astype(np.float64) / 64.0)


# ---------------------------------------------------------------- relu^2
def test_relu2_cases(oracle_mod):
    g = np.array([-3.0, -0.0, 0.0, 1e-30, 2.0, 0.5, 1.5], np.float32)
    u = np.array([5.0, 7.0, -2.0, 1.0, -3.0, 4.0, 1e-20], np.float32)
    h = oracle_mod.relu2(g, u)
    assert h[0] == 0 and h[1] == 0 and h[2] == 0
    assert h[4] == np.float32(-12.0) and h[5] == np.float32(1.0)
    for i in range(len(g)):
        r = Fraction(float(g[i])) if g[i] > 0 else Fraction(0)
        want = ieee.rn32(ieee.rn32(r * r) * Fraction(float(u[i])))
        assert Fraction(float(h[i])) == want
    h64 = oracle_mod.relu2(g.astype(np.float64), u.astype(np.float64), exact=True)
    for i in range(len(g)):
        r = max(float(g[i]), 0.0)
        assert h64[i] == r * r * float(u[i])


def test_relu2_bound(oracle_mod):
    rng = np.random.default_rng(12)
    g = rng.standard_normal(1000).astype(np.float32)
    u = rng.standard_normal(1000).astype(np.float32)
    h = oracle_mod.relu2(g, u).astype(np.float64)
    ex = np.maximum(g.astype(np.float64), 0) ** 2 * u.astype(np.float64)
    nz = ex != 0
    assert np.all(h[~nz] == 0)
    assert np.max(np.abs(h[nz] - ex[nz]) / np.abs(ex[nz])) <= 2 * 2.0 ** -24 * 1.0001
