"""GPU parity of the sub-layer RMSNorm folded into the quantization
(tq_rmsnorm_act_quant, tq_rmsnorm_quant_gemv) against the CPU oracle.

The codes (int8) and the int32 sums are exact decisions and must be
bit-exact.  The scale s_x = (a'/127) * r carries r = 1/sqrt(mean(x^2) + eps),
whose fp64 sum of squares is ordered differently on the GPU (per-thread
runs, wave trees) and in the oracle (one running sum); r is rounded once to
fp32, so s_x agrees bit for bit except when the two fp64 sums straddle an
fp32 rounding boundary: the test allows one fp32 ulp.  y = acc * (s_w * s_x)
is then within 1e-6 relative of the oracle's exact (fp64) value.

Cases: the o_proj and down shapes of a 2B-4T layer, the 70B-class down
shape the benchmark times, ragged and tiny rows, K past the single-pass
limit (two launches), N = 0, negative RMSNorm weights, a zero row, many
rows through tq_rmsnorm_act_quant, fused vs two-call agreement, and
repeatability.
"""
import sys

import numpy as np
import pytest

import workloads

pytestmark = pytest.mark.gpu

REL_TOL = 1e-6
EPS = 1e-5


@pytest.fixture(scope="module")
def env():
    import torch
    import bit_gemv_tq_amd as tq
    import oracle
    return torch, tq, oracle


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_bf16(a):
    return (np.asarray(a, np.float32).view(np.uint32) >> 16).astype(np.uint16)


def row_data(K, M, dtype, seed):
    """(host x, host gamma) in the oracle's form: bf16 bit patterns or fp32."""
    rng = np.random.default_rng(seed)
    g = (1.0 + 0.25 * rng.standard_normal(K)).astype(np.float32)
    g[::9] *= -1.0
    if dtype == "bf16":
        return workloads.activations_bf16(M, K, seed=seed, outliers=True), to_bf16(g)
    return workloads.normal_f32(M, K, seed=seed, outliers=True) * np.float32(0.7), g


def dev(torch, a, dtype):
    if dtype == "bf16":
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(a).cuda()


def check_scale(got, ref):
    got = np.asarray(got, np.float32).reshape(-1)
    ref = np.asarray(ref, np.float32).reshape(-1)
    assert np.all(np.abs(got.astype(np.float64) - ref) <= np.spacing(ref)), (got, ref)


def check_y(y, acc_ref, s_w, s_x_ref):
    """y against the exact value with the oracle's scale: within 1e-6."""
    exact = acc_ref.astype(np.float64) * float(np.float32(s_w)) * float(s_x_ref)
    err = np.abs(y.astype(np.float64) - exact)
    assert np.all(err <= REL_TOL * np.abs(exact)), float(
        np.max(err / np.maximum(np.abs(exact), 1e-300)))


@pytest.mark.parametrize("M,K", [(1, 16), (1, 2560), (4, 6912), (64, 2560),
                                 (2, 28672), (3, 32768), (2, 32784), (1, 131072)])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_rmsnorm_act_quant(env, M, K, dtype):
    torch, tq, oracle = env
    say(f"rmsnorm_act_quant {dtype} M={M} K={K}")
    xh, gh = row_data(K, M, dtype, seed=M * 7 + K)
    x, g = dev(torch, xh, dtype).reshape(M, K), dev(torch, gh, dtype)
    xq, xs = tq.tq_rmsnorm_act_quant(x, g, EPS)
    torch.cuda.synchronize()
    q_ref, s_ref = oracle.rmsnorm_act_quant(xh.reshape(M, K), gh, EPS, dtype)
    np.testing.assert_array_equal(xq.cpu().numpy(), q_ref)
    check_scale(xs.cpu().numpy(), s_ref)


# (N, K): 2B-4T o_proj and down, the 70B-class down shape, ragged and tiny
# rows, K past the single-pass limit, N = 0, and (20480, 20480), where each
# 256-lane team (two per block) walks 10 rows, so its per-row sum slots are
# reused across the periodic barrier, and (16384, 14336), whose persistent
# grid is capped at the two blocks per CU the 128-lane form's registers allow
SHAPES = [(2560, 2560), (2560, 6912), (8192, 28672), (20, 48), (100, 4112),
          (4, 16), (8, 32784), (0, 2560), (20480, 20480), (16384, 14336)]


@pytest.mark.parametrize("N,K", SHAPES)
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_rmsnorm_quant_gemv(env, N, K, dtype):
    torch, tq, oracle = env
    say(f"rmsnorm_quant_gemv {dtype} N={N} K={K}")
    codes = workloads.ternary_codes(N, K, seed=N * 3 + K + 1)
    ref = oracle.pack(codes)
    packed = torch.from_numpy(ref).cuda()
    xh, gh = row_data(K, 1, dtype, seed=K + 17)
    x, g = dev(torch, xh, dtype)[0], dev(torch, gh, dtype)
    s_w = np.float32(0.023)
    acc = torch.full((N,), 7, dtype=torch.int32, device="cuda")
    xq = torch.empty(K, dtype=torch.int8, device="cuda")
    xs = torch.empty(1, dtype=torch.float32, device="cuda")
    y = tq.tq_rmsnorm_quant_gemv(x, g, packed, s_w, eps=EPS, acc=acc, xq=xq, x_scale=xs)
    torch.cuda.synchronize()
    q_ref, s_ref = oracle.rmsnorm_act_quant(xh.reshape(1, K), gh, EPS, dtype)
    np.testing.assert_array_equal(xq.cpu().numpy(), q_ref[0])
    check_scale(xs.cpu().numpy(), s_ref)
    if N == 0:
        return
    acc_ref = oracle.ternary_matmul(ref, q_ref, N)[0]
    np.testing.assert_array_equal(acc.cpu().numpy(), acc_ref)
    check_y(y.cpu().numpy(), acc_ref, s_w, s_ref[0])


@pytest.mark.parametrize("N,K", [(2560, 2560), (2560, 6912), (8192, 28672), (8, 32784)])
def test_fused_matches_two_calls(env, N, K):
    # one launch vs tq_rmsnorm_act_quant + tq_gemv: codes and sums equal; the
    # scale (and so y) within the last bit (sums of squares ordered apart)
    torch, tq, oracle = env
    say(f"rmsnorm fused vs two calls N={N} K={K}")
    codes = workloads.ternary_codes(N, K, seed=N + K + 5)
    packed = torch.from_numpy(oracle.pack(codes)).cuda()
    xh, gh = row_data(K, 1, "bf16", seed=K + 23)
    x, g = dev(torch, xh, "bf16")[0], dev(torch, gh, "bf16")
    acc1 = torch.empty(N, dtype=torch.int32, device="cuda")
    acc2 = torch.empty(N, dtype=torch.int32, device="cuda")
    xq1 = torch.empty(K, dtype=torch.int8, device="cuda")
    xs1 = torch.empty(1, dtype=torch.float32, device="cuda")
    y1 = tq.tq_rmsnorm_quant_gemv(x, g, packed, 0.02, eps=EPS, acc=acc1, xq=xq1, x_scale=xs1)
    xq2, xs2 = tq.tq_rmsnorm_act_quant(x, g, EPS)
    y2 = tq.tq_gemv(packed, 0.02, xq2[0], xs2, acc=acc2)
    torch.cuda.synchronize()
    assert torch.equal(xq1, xq2[0])
    assert torch.equal(acc1, acc2)
    check_scale(xs1.cpu().numpy(), xs2.cpu().numpy())
    a = y1.cpu().numpy().astype(np.float64)
    b = y2.cpu().numpy().astype(np.float64)
    assert np.all(np.abs(a - b) <= 2 * REL_TOL * np.abs(b))


def test_zero_row_and_repeatability(env):
    torch, tq, oracle = env
    say("rmsnorm zero row, repeatability")
    N, K = 2560, 6912
    codes = workloads.ternary_codes(N, K, seed=99)
    packed = torch.from_numpy(oracle.pack(codes)).cuda()
    g = torch.ones(K, dtype=torch.float32, device="cuda")
    x0 = torch.zeros(K, dtype=torch.float32, device="cuda")
    xq = torch.empty(K, dtype=torch.int8, device="cuda")
    xs = torch.empty(1, dtype=torch.float32, device="cuda")
    y = tq.tq_rmsnorm_quant_gemv(x0, g, packed, 0.02, eps=EPS, xq=xq, x_scale=xs)
    torch.cuda.synchronize()
    assert int(xq.abs().sum()) == 0
    assert int((y != 0).sum()) == 0
    _, s_ref = oracle.rmsnorm_act_quant(np.zeros((1, K), np.float32),
                                        np.ones(K, np.float32), EPS, "f32")
    check_scale(xs.cpu().numpy(), s_ref)
    xh, gh = row_data(K, 1, "bf16", seed=5)
    x, gb = dev(torch, xh, "bf16")[0], dev(torch, gh, "bf16")
    first = tq.tq_rmsnorm_quant_gemv(x, gb, packed, 0.02, eps=EPS)
    for _ in range(3):
        again = tq.tq_rmsnorm_quant_gemv(x, gb, packed, 0.02, eps=EPS)
        torch.cuda.synchronize()
        assert torch.equal(again.view(torch.int32), first.view(torch.int32))
