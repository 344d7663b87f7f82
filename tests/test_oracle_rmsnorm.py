"""Pins of the oracle's sub-layer RMSNorm folded into the per-token
quantization (page "Feature request: BitNet 1.58-bit ternary inference on
ROCm (gfx1151)", section "Architecture": norms before o_proj and down_proj).

RMSNorm(x)_k = x_k * gamma_k / sqrt(mean(x^2) + eps).  The oracle returns the
absmax codes of u = x*gamma and s_x = (a'/127) * r; these pins check it
against the plain definition in fp64 (dequantized values within half a step
of RMSNorm(x)*gamma), a closed form, the scale invariance that defines
RMSNorm, the zero row, and the argument checks.
"""
import numpy as np
import pytest

import oracle
import workloads


def rms_f64(x, g, eps):
    x = x.astype(np.float64)
    return x * g.astype(np.float64) / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)


def bf16(a):
    return (np.asarray(a, np.float32).view(np.uint32) >> 16).astype(np.uint16)


def from_bf16(b):
    return (b.astype(np.uint32) << 16).view(np.float32)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("K", [16, 2560, 6912])
def test_dequantized_close_to_definition(dtype, K):
    rng = np.random.default_rng(K)
    M = 3
    xf = rng.standard_normal((M, K)).astype(np.float32) * np.float32(3.0)
    gf = (1.0 + 0.3 * rng.standard_normal(K)).astype(np.float32)
    gf[::7] *= -1.0                               # negative weights too
    if dtype == "bf16":
        xb, gb = bf16(xf), bf16(gf)
        xf, gf = from_bf16(xb), from_bf16(gb)
        q, s = oracle.rmsnorm_act_quant(xb, gb, 1e-6, "bf16")
    else:
        q, s = oracle.rmsnorm_act_quant(xf, gf, 1e-6, "f32")
    ref = rms_f64(xf, gf, 1e-6)
    deq = q.astype(np.float64) * s.astype(np.float64)[:, None]
    # half a quantization step, plus the fp32 roundings of u, inv, s_x, r
    tol = s.astype(np.float64)[:, None] * (0.5 + 1e-4)
    assert np.all(np.abs(deq - ref) <= tol)
    # the largest |RMSNorm(x)*gamma| of each row lands on +-127
    assert np.all(np.abs(q).max(axis=1) == 127)


def test_closed_form():
    # x = (3, 4, 0, ...), gamma = 1, K = 16: mean(x^2) = 25/16
    x = np.zeros((1, 16), np.float32)
    x[0, :2] = (3.0, 4.0)
    q, s = oracle.rmsnorm_act_quant(x, np.ones(16, np.float32), 1e-6, "f32")
    assert q[0, :2].tolist() == [95, 127]         # rne(3 * 127/4) = rne(95.25)
    assert np.all(q[0, 2:] == 0)
    want = (4.0 / 127.0) / np.sqrt(25.0 / 16.0 + 1e-6)
    assert abs(float(s[0]) - want) <= 2 * np.spacing(np.float32(want))


def test_scale_invariance():
    # RMSNorm(c x) = RMSNorm(x): same codes, same scale (up to the eps term
    # and one rounding each of r and s_x)
    rng = np.random.default_rng(5)
    x = rng.standard_normal((2, 2560)).astype(np.float32)
    g = (1.0 + 0.2 * rng.standard_normal(2560)).astype(np.float32)
    eps = 1e-9
    q1, s1 = oracle.rmsnorm_act_quant(x, g, eps, "f32")
    ms = np.mean(x.astype(np.float64) ** 2, axis=1)
    for c in (np.float32(256.0), np.float32(2.0 ** -6)):
        q2, s2 = oracle.rmsnorm_act_quant(x * c, g, eps, "f32")
        assert np.array_equal(q1, q2)
        # roundings of s_x and r on both sides, plus the eps term's share
        rtol = 4 * 2.0 ** -24 + eps / (2 * ms * min(1.0, float(c) ** 2))
        assert np.all(np.abs(s2.astype(np.float64) / s1 - 1.0) <= rtol)


def test_zero_row():
    x = np.zeros((1, 64), np.float32)
    q, s = oracle.rmsnorm_act_quant(x, np.ones(64, np.float32), 1e-5, "f32")
    assert np.all(q == 0)
    want = np.float32(np.float32(1e-5) / np.float32(127.0)) * np.float32(1.0 / np.sqrt(np.float64(np.float32(1e-5))))
    assert s[0] == want


def test_codes_are_those_of_x_times_gamma():
    # the codes do not depend on r: they equal plain absmax quantization of
    # the fp32 products (an independent NumPy rendering of that rule)
    xb = workloads.activations_bf16(2, 2560, seed=11, outliers=True)
    rng = np.random.default_rng(12)
    gb = bf16((1.0 + 0.3 * rng.standard_normal(2560)).astype(np.float32))
    q, _ = oracle.rmsnorm_act_quant(xb, gb, 1e-6, "bf16")
    u = from_bf16(xb) * from_bf16(gb)
    a = np.maximum(np.abs(u).max(axis=1, keepdims=True), np.float32(1e-5))
    inv = (np.float32(127.0) / a).astype(np.float32)
    want = np.clip(np.rint((u * inv).astype(np.float32)), -127, 127).astype(np.int8)
    assert np.array_equal(q, want)


def test_argument_checks():
    x = np.ones((1, 16), np.float32)
    with pytest.raises(oracle.OracleError):
        oracle.rmsnorm_act_quant(x, np.ones(16, np.float32), 0.0, "f32")   # eps > 0
    with pytest.raises(ValueError):
        oracle.rmsnorm_act_quant(x, np.ones(8, np.float32), 1e-5, "f32")


def test_folded_codes_equal_normalize_then_quantize():
    """The folded reading (codes of x*gamma, the RMS factor r in the scale)
    against the plain order -- normalize first, n = (x*r)*gamma in fp32, then
    quantize n by its own absmax -- on 60 seeded bf16 rows with outliers at
    the hidden sizes K = 2560, 6912, 28672: every code is the same, and the
    two scales agree to a few fp32 ulps.  Absmax quantization is scale
    invariant in exact arithmetic; this pins that the fp32 roundings of
    either order do not move a code on these rows."""
    total = 0
    for K in (2560, 6912, 28672):
        for r in range(20):
            xb = workloads.activations_bf16(1, K, seed=7000 + K + r, outliers=True)
            rng = np.random.default_rng(8000 + K + r)
            gb = bf16((1.0 + 0.1 * rng.standard_normal(K)).astype(np.float32))
            q, s = oracle.rmsnorm_act_quant(xb, gb, 1e-5, "bf16")
            x, g = from_bf16(xb)[0], from_bf16(gb)
            ms = np.mean(x.astype(np.float64) ** 2) + np.float64(np.float32(1e-5))
            r32 = np.float32(1.0 / np.sqrt(ms))
            n = ((x * r32).astype(np.float32) * g).astype(np.float32)
            qp, sp = oracle.act_quant(n[None, :], "f32")
            np.testing.assert_array_equal(qp, q)
            assert abs(float(sp[0]) - float(s[0])) <= 4 * np.spacing(np.float32(s[0]))
            total += K
    assert total == 762880
