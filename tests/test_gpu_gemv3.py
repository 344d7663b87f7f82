"""GPU parity of the five-weights-per-byte layout (tq_pack3, tq_gemv3)
against the CPU oracle.

Packed bytes, int32 sums and fp32 outputs are bit-exact: the sums against
the oracle's exact product over its own unpacking of the bytes, y against
the oracle's fp32 rescale, and both against tq_gemv on the two-bit packing of
the same weights.  Shapes: tiny and ragged N (N % 5 != 0, padding rows), the
2B-4T projections, the 70B-class shapes the benchmark times, the largest K,
and one lane-team width per K range.
"""
import sys

import numpy as np
import pytest

import workloads

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def env():
    import torch
    import bit_gemv_tq_amd as tq
    import oracle
    return torch, tq, oracle


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.mark.parametrize("N,K", [(1, 16), (5, 16), (7, 48), (13, 272), (640, 2560),
                                 (6912, 2560), (2560, 6912)])
def test_pack3(env, N, K):
    torch, tq, oracle = env
    say(f"pack3 N={N} K={K}")
    codes = workloads.ternary_codes(N, K, seed=N * 7 + K)
    got = tq.tq_pack3(torch.from_numpy(codes).cuda())
    torch.cuda.synchronize()
    np.testing.assert_array_equal(got.cpu().numpy(), oracle.pack3(codes))


def test_pack3_bad_value_is_reserved(env):
    torch, tq, oracle = env
    w = torch.zeros(5, 16, dtype=torch.int8)
    w[3, 7] = 2
    got = tq.tq_pack3(w.cuda()).cpu().numpy()
    assert got[0, 7] == 1                      # reserved byte
    with pytest.raises(oracle.OracleError):
        oracle.unpack3(got, 5)


# (N, K): tiny, ragged N, one shape per lane-team width (16..256 lanes), the
# 2B-4T projections, the 70B-class shapes, the largest K
SHAPES = [(3, 16), (7, 48), (13, 272), (101, 1040), (64, 4096), (40, 8192),
          (20, 16384), (2560, 2560), (640, 2560), (6912, 2560), (2560, 6912),
          (8192, 28672), (28672, 8192), (9, 32768)]


@pytest.mark.parametrize("N,K", SHAPES)
def test_gemv3(env, N, K):
    torch, tq, oracle = env
    say(f"gemv3 N={N} K={K}")
    codes = workloads.ternary_codes(N, K, seed=N * 11 + K)
    w = torch.from_numpy(codes).cuda()
    p3 = tq.tq_pack3(w)
    p2 = tq.tq_pack(torch.cat([w, torch.zeros((-N) % 4, K, dtype=torch.int8, device="cuda")]))
    xb = workloads.activations_bf16(1, K, seed=K + 29, outliers=True)
    x = torch.from_numpy(xb.view(np.int16)).view(torch.bfloat16).cuda()
    xq, xs = tq.tq_act_quant(x)
    s_w = np.float32(0.019)
    acc = torch.full((N,), 7, dtype=torch.int32, device="cuda")
    y = tq.tq_gemv3(p3, s_w, xq[0], xs, N, acc=acc)
    acc2 = torch.empty(p2.shape[0] * 4, dtype=torch.int32, device="cuda")
    y2 = tq.tq_gemv(p2, s_w, xq[0], xs, acc=acc2)
    torch.cuda.synchronize()
    q_ref, s_ref = oracle.act_quant(xb.reshape(1, K), "bf16")
    ref_bytes = oracle.pack3(codes)
    np.testing.assert_array_equal(p3.cpu().numpy(), ref_bytes)
    unpacked = oracle.unpack3(ref_bytes, N)
    pad = (-N) % 4
    acc_ref, y32 = oracle.gemv(oracle.pack(np.vstack([unpacked, np.zeros((pad, K), np.int8)])),
                               s_w, q_ref, s_ref, N + pad)
    np.testing.assert_array_equal(acc.cpu().numpy(), acc_ref[0, :N])
    np.testing.assert_array_equal(y.cpu().numpy().view(np.uint32), y32[0, :N].view(np.uint32))
    assert torch.equal(acc, acc2[:N])
    assert torch.equal(y.view(torch.int32), y2[:N].view(torch.int32))


def test_gemv3_empty_and_repeatable(env):
    torch, tq, _ = env
    say("gemv3 N=0, repeatability")
    xq = torch.zeros(64, dtype=torch.int8, device="cuda")
    xs = torch.ones(1, dtype=torch.float32, device="cuda")
    empty = torch.empty(0, 64, dtype=torch.uint8, device="cuda")
    assert tq.tq_gemv3(empty, 0.02, xq, xs, 0).numel() == 0
    codes = workloads.ternary_codes(2560, 6912, seed=5)
    p3 = tq.tq_pack3(torch.from_numpy(codes).cuda())
    xb = workloads.activations_bf16(1, 6912, seed=6, outliers=True)
    x = torch.from_numpy(xb.view(np.int16)).view(torch.bfloat16).cuda()
    xq, xs = tq.tq_act_quant(x)
    first = tq.tq_gemv3(p3, 0.02, xq[0], xs, 2560)
    for _ in range(3):
        again = tq.tq_gemv3(p3, 0.02, xq[0], xs, 2560)
        torch.cuda.synchronize()
        assert torch.equal(again.view(torch.int32), first.view(torch.int32))
