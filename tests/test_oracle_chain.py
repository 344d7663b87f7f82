"""Pins for the oracle's decode-step chain (composition of pinned primitives).

The chain's wiring and its unit-activation-scale reading are pinned by
structural cases: zeroing one projection's weights must silence exactly the
stages that depend on it, negating up or down must negate h bit for bit, and
a power-of-two rescale of the input must leave every stage unchanged.
"""
import numpy as np

import workloads


def make_layer(oracle_mod, H=16, Q=16, KV=8, I=24, seed=0, zero=(), neg=()):
    shapes = {"q": (Q, H), "k": (KV, H), "v": (KV, H), "o": (H, Q),
              "gate": (I, H), "up": (I, H), "down": (H, I)}
    layer = {}
    for t, (name, (N, K)) in enumerate(shapes.items()):
        w = workloads.ternary_codes(N, K, seed=seed * 10 + t)
        if name in zero:
            w[...] = 0
        if name in neg:
            w = -w
        layer[name] = (oracle_mod.pack(w), workloads.tensor_scale(t), N)
    return layer


def test_chain_runs_and_stays_nonzero(oracle_mod):
    layers = [make_layer(oracle_mod, seed=s) for s in range(6)]
    h0 = workloads.activations_bf16(1, 16, seed=1, outliers=True)
    h, st = oracle_mod.decode_chain(layers, h0, keep_stages=True)
    assert h.shape == (1, 16) and np.isfinite(h).all()
    for s in st:
        assert np.abs(s["h"]).max() > 0
        assert s["q8_in"].dtype == np.int8 and np.abs(s["q8_in"]).max() == 127


def test_zero_weights_silence_dependents(oracle_mod):
    h0 = workloads.activations_bf16(1, 16, seed=2)
    for name in ("q", "o", "gate", "up", "down"):
        st = oracle_mod.decode_layer(make_layer(oracle_mod, zero=(name,)), h0, "bf16")
        assert not st["h"].any(), name
    base = oracle_mod.decode_layer(make_layer(oracle_mod), h0, "bf16")
    for name in ("k", "v"):                   # k, v feed nothing on this path
        st = oracle_mod.decode_layer(make_layer(oracle_mod, zero=(name,)), h0, "bf16")
        np.testing.assert_array_equal(st["h"], base["h"])
        assert not st[name].any()


def test_sign_flips(oracle_mod):
    h0 = workloads.activations_bf16(1, 16, seed=3)
    base = oracle_mod.decode_layer(make_layer(oracle_mod), h0, "bf16")
    for name in ("up", "down"):
        st = oracle_mod.decode_layer(make_layer(oracle_mod, neg=(name,)), h0, "bf16")
        np.testing.assert_array_equal(st["h"], -base["h"])


def test_input_scale_invariance(oracle_mod):
    # Re-quantization with the unit activation scale makes each layer depend
    # only on the direction of its input.
    layer = make_layer(oracle_mod)
    x = workloads.normal_f32(1, 16, seed=4)
    a = oracle_mod.decode_layer(layer, x, "f32")
    b = oracle_mod.decode_layer(layer, (x * np.float32(8.0)).astype(np.float32), "f32")
    for key in ("q8_in", "q", "o", "f", "h"):
        np.testing.assert_array_equal(a[key], b[key])


def test_stage_shapes_2b4t(oracle_mod):
    layer = {}
    for t, (name, (N, K)) in enumerate(workloads.LAYER_2B4T.items()):
        w = workloads.ternary_codes(N, K, seed=t)
        layer[name] = (oracle_mod.pack(w), workloads.tensor_scale(t), N)
    h0 = workloads.activations_bf16(1, workloads.HIDDEN, seed=5, outliers=True)
    st = oracle_mod.decode_layer(layer, h0, "bf16")
    assert st["q"].shape == (1, 2560) and st["k"].shape == (1, 640)
    assert st["f"].shape == (1, 6912) and st["h"].shape == (1, 2560)
    assert 0.01 < np.abs(st["h"]).max() < 100
