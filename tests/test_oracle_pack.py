"""Pins for the oracle's packing (pack / unpack).

Packed shapes come from the page "Feature request: BitNet 1.58-bit ternary
inference on ROCm (gfx1151)", section "Weight mapping (bitnet-b1.58-2B-4T)"
(tests/golden/weight_map_2b4t.json); the bit assignment is the reading
fixed in tests/golden/pack_example.json, derived by hand.
"""
import itertools
import json
import os

import numpy as np
import pytest

import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_pack_hand_example(oracle_mod):
    d = json.load(open(os.path.join(GOLDEN, "pack_example.json")))
    w = np.array(d["w"], np.int8)
    got = oracle_mod.pack(w)
    np.testing.assert_array_equal(got, np.array(d["packed"], np.uint8))
    np.testing.assert_array_equal(oracle_mod.unpack(got, d["N"]), w)


def test_pack_exhaustive_bytes(oracle_mod):
    # Every one of the 3^4 = 81 columns of four ternary rows maps to a
    # distinct byte, never uses code 3, and unpacks to itself.
    cols = np.array(list(itertools.product((-1, 0, 1), repeat=4)), np.int8)
    w = cols.T.copy()                        # [4, 81]: N=4, K=81
    p = oracle_mod.pack(w)
    assert p.shape == (1, 81)
    assert len(set(p[0].tolist())) == 81
    for j in range(4):
        assert np.all(((p >> (2 * j)) & 3) != 3)
    np.testing.assert_array_equal(oracle_mod.unpack(p, 4), w)
    # Per-field value: field j of each byte is w[j] + 1.
    for j in range(4):
        np.testing.assert_array_equal((p[0] >> (2 * j)) & 3, cols[:, j] + 1)


@pytest.mark.parametrize("N,K", [(4, 1), (8, 17), (64, 33), (12, 160)])
def test_pack_roundtrip_random(oracle_mod, N, K):
    w = workloads.ternary_codes(N, K, seed=N * 1000 + K)
    p = oracle_mod.pack(w)
    assert p.shape == (N // 4, K) and p.dtype == np.uint8
    np.testing.assert_array_equal(oracle_mod.unpack(p, N), w)


def test_weight_map_shapes(oracle_mod):
    d = json.load(open(os.path.join(GOLDEN, "weight_map_2b4t.json")))
    for name, e in d["projections"].items():
        N, K = e["unpacked"]
        w = np.zeros((N, K), np.int8)
        p = oracle_mod.pack(w)
        assert list(p.shape) == e["packed"], name
        # 2B-4T hyper-parameters agree with the synthetic workload shapes.
        short = name.split("_")[0]
        assert workloads.LAYER_2B4T[short] == (N, K), name
    h = d["hyper"]
    assert h["hidden_size"] == workloads.HIDDEN
    assert h["intermediate_size"] == workloads.INTERMEDIATE
    assert h["num_kv_heads"] * h["head_dim"] == workloads.KV_DIM


def test_pack_rejects_bad_input(oracle_mod):
    with pytest.raises(oracle_mod.OracleError):
        oracle_mod.pack(np.full((4, 2), 2, np.int8))
    with pytest.raises(oracle_mod.OracleError):
        oracle_mod.pack(np.zeros((6, 2), np.int8))
    bad = np.array([[0b11]], np.uint8)            # code 3 in field 0
    with pytest.raises(oracle_mod.OracleError):
        oracle_mod.unpack(bad, 4)


def test_pack_empty(oracle_mod):
    assert oracle_mod.pack(np.zeros((0, 5), np.int8)).shape == (0, 5)
    assert oracle_mod.pack(np.zeros((8, 0), np.int8)).shape == (2, 0)
