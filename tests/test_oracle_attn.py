"""Pins for the oracle's decode attention (one query token, grouped-query
heads, bf16 KV cache): closed forms (one token, identical keys, zero query,
per-group constant values), invariances (token permutation, a common key
shift), a dominant key, and PyTorch's own scaled-dot-product attention in
float64 on the CPU as an independent library routine.
"""
import numpy as np
import pytest


def bf16(x):
    """fp32 -> bf16 bits by truncation (test data only)."""
    return (np.asarray(x, np.float32).view(np.uint32) >> 16).astype(np.uint16)


def widen(b):
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def rand_case(L, H=20, Hkv=5, D=128, seed=0):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((H, D)).astype(np.float32)
    k = bf16(rng.standard_normal((L, Hkv, D)))
    v = bf16(rng.standard_normal((L, Hkv, D)))
    return q, k, v, np.float32(1.0 / np.sqrt(D))


def test_single_token_returns_its_value(oracle_mod):
    q, k, v, sc = rand_case(1, seed=1)
    o = oracle_mod.attn_decode(q, k, v, sc)
    for h in range(20):
        np.testing.assert_array_equal(o[h], widen(v[0, h // 4]))


def test_identical_keys_or_zero_query_average_values(oracle_mod):
    q, k, v, sc = rand_case(37, seed=2)
    k[:] = k[0]                                     # every key the same
    o = oracle_mod.attn_decode(q, k, v, sc)
    for h in range(20):
        np.testing.assert_allclose(o[h], widen(v[:, h // 4]).mean(axis=0), rtol=0, atol=1e-14)
    q, k, v, sc = rand_case(37, seed=3)
    o = oracle_mod.attn_decode(np.zeros_like(q), k, v, sc)
    np.testing.assert_allclose(o[7], widen(v[:, 1]).mean(axis=0), rtol=0, atol=1e-14)


def test_group_mapping(oracle_mod):
    # value rows constant per kv head g (= g + 1): head h must read group h // 4
    q, k, v, sc = rand_case(50, seed=4)
    for g in range(5):
        v[:, g, :] = bf16(np.full((50, 128), g + 1.0))
    o = oracle_mod.attn_decode(q, k, v, sc)
    for h in range(20):
        np.testing.assert_allclose(o[h], h // 4 + 1.0, rtol=0, atol=1e-13)


def test_permutation_and_key_shift_invariance(oracle_mod):
    q, k, v, sc = rand_case(64, seed=5)
    o = oracle_mod.attn_decode(q, k, v, sc)
    perm = np.random.default_rng(6).permutation(64)
    np.testing.assert_allclose(oracle_mod.attn_decode(q, k[perm], v[perm], sc), o,
                               rtol=0, atol=1e-13)
    # small-integer keys shifted by a common small-integer vector stay exact in
    # bf16; every score moves by the same q.c, so softmax is unchanged
    rng = np.random.default_rng(7)
    ki = rng.integers(-4, 5, (64, 5, 128)).astype(np.float32)
    c = rng.integers(-3, 4, (1, 5, 128)).astype(np.float32)
    qs = (rng.integers(-2, 3, (20, 128)) / 8).astype(np.float32)
    a = oracle_mod.attn_decode(qs, bf16(ki), v, sc)
    b = oracle_mod.attn_decode(qs, bf16(ki + c), v, sc)
    np.testing.assert_allclose(a, b, rtol=0, atol=1e-12)


def test_dominant_key(oracle_mod):
    q, k, v, sc = rand_case(200, seed=8)
    j = 123
    q[0] = widen(k[j, 0]).astype(np.float32) * 4.0   # score gap of ~ 4*128*sc
    o = oracle_mod.attn_decode(q, k, v, sc)
    np.testing.assert_allclose(o[0], widen(v[j, 0]), rtol=0, atol=1e-6)


def test_matches_torch_sdpa_float64(oracle_mod):
    import torch
    import torch.nn.functional as F
    for L, seed in ((5, 9), (300, 10), (2048, 11)):
        q, k, v, sc = rand_case(L, seed=seed)
        o = oracle_mod.attn_decode(q, k, v, sc)
        qt = torch.from_numpy(q.astype(np.float64)).reshape(1, 20, 1, 128)
        kt = torch.from_numpy(widen(k)).permute(1, 0, 2).reshape(1, 5, L, 128)
        vt = torch.from_numpy(widen(v)).permute(1, 0, 2).reshape(1, 5, L, 128)
        kt = kt.repeat_interleave(4, dim=1).contiguous()
        vt = vt.repeat_interleave(4, dim=1).contiguous()
        ref = F.scaled_dot_product_attention(qt, kt, vt, scale=float(sc))
        np.testing.assert_allclose(o, ref.reshape(20, 128).numpy(), rtol=0, atol=1e-12)


def test_bad_shapes(oracle_mod):
    q, k, v, sc = rand_case(4, seed=12)
    with pytest.raises(oracle_mod.OracleError):
        oracle_mod.attn_decode(q[:, :64], k, v, sc)
    with pytest.raises(oracle_mod.OracleError):
        oracle_mod.attn_decode(q, k[:0], v[:0], sc)
