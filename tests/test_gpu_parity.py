"""GPU parity: every C-ABI call against the CPU oracle on the same seeded
inputs.  Integer results (packed bytes, int8 activations, int32 sums) must be
bit-exact; fp32 results must be within 1e-6 relative of the oracle's exact
(fp64) value and, with the fixed operation order of the rescale, are also
expected bit-exact against the oracle's fp32 path.

Sizes span several tiles with ragged tails (N/4 not a multiple of a block's
rows, K/16 not a multiple of a lane group), the maximum K, empty shapes, and
the full 2B-4T and 70B-class layer shapes in the launch configuration the
benchmark times.
"""
import sys

import numpy as np
import pytest

import workloads

pytestmark = pytest.mark.gpu

REL_TOL = 1e-6


@pytest.fixture(scope="module")
def env():
    import torch
    import bit_gemv_tq_amd as tq
    import oracle
    return torch, tq, oracle


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev_packed(env, codes):
    """Pack on the GPU and check the bytes against the oracle's packing."""
    torch, tq, oracle = env
    w = torch.from_numpy(codes).cuda()
    packed = tq.tq_pack(w)
    ref = oracle.pack(codes)
    got = packed.cpu().numpy()
    np.testing.assert_array_equal(got, ref)
    return packed, ref


def quantized(env, xbits, M, K):
    """bf16 activations -> (GPU xq, GPU s_x), checked bit-exact vs oracle."""
    torch, tq, oracle = env
    x = torch.from_numpy(xbits.view(np.int16)).view(torch.bfloat16).cuda().reshape(M, K)
    xq, xs = tq.tq_act_quant(x)
    q_ref, s_ref = oracle.act_quant(xbits.reshape(M, K), "bf16")
    np.testing.assert_array_equal(xq.cpu().numpy(), q_ref)
    np.testing.assert_array_equal(xs.cpu().numpy().view(np.uint32),
                                  s_ref.view(np.uint32))
    return xq, xs, q_ref, s_ref


def check_y(y_gpu, y32_ref, y64_ref):
    y = y_gpu.reshape(y32_ref.shape).astype(np.float64)
    err = np.abs(y - y64_ref)
    assert np.all(err <= REL_TOL * np.abs(y64_ref)), float(
        np.max(err / np.maximum(np.abs(y64_ref), 1e-300)))
    np.testing.assert_array_equal(y_gpu.reshape(y32_ref.shape).view(np.uint32),
                                  y32_ref.view(np.uint32))


# ------------------------------------------------------------------ pack
@pytest.mark.parametrize("N,K", [(4, 16), (8, 32), (20, 48), (100, 1008),
                                 (640, 2560), (6912, 2560), (2560, 6912)])
def test_pack(env, N, K):
    say(f"pack N={N} K={K}")
    dev_packed(env, workloads.ternary_codes(N, K, seed=N + K))


def test_pack_reserved_code(env):
    torch, tq, _ = env
    w = torch.zeros(4, 16, dtype=torch.int8)
    w[2, 5] = 7
    w[0, 0] = -1
    p = tq.tq_pack(w.cuda()).cpu().numpy()
    assert (p[0, 5] >> 4) & 3 == 3           # row 2 = plane 2 of packed row 0
    assert p[0, 0] & 3 == 0 and (p[0, 0] >> 2) & 3 == 1


# ------------------------------------------------------------------ act quant
@pytest.mark.parametrize("M,K", [(1, 16), (1, 2560), (4, 2560), (16, 6912),
                                 (64, 2560), (3, 28672), (1, 131072)])
def test_act_quant_bf16(env, M, K):
    say(f"act_quant bf16 M={M} K={K}")
    xb = workloads.activations_bf16(M, K, seed=M * 7 + K, outliers=True)
    quantized(env, xb, M, K)


@pytest.mark.parametrize("M,K", [(1, 2560), (5, 6912), (64, 160)])
def test_act_quant_f32(env, M, K):
    torch, tq, oracle = env
    say(f"act_quant f32 M={M} K={K}")
    x = workloads.normal_f32(M, K, seed=K + M, outliers=True) * np.float32(0.37)
    xq, xs = tq.tq_act_quant(torch.from_numpy(x).cuda())
    q_ref, s_ref = oracle.act_quant(x, "f32")
    np.testing.assert_array_equal(xq.cpu().numpy(), q_ref)
    np.testing.assert_array_equal(xs.cpu().numpy(), s_ref)


def test_act_quant_exhaustive_bf16(env):
    # Every finite bf16 value, quantized against 64 different absmax values
    # (tiny to huge, including below the 1e-5 floor).
    torch, tq, oracle = env
    bits = np.arange(1 << 16, dtype=np.uint32)
    xs = (bits << 16).view(np.float32)
    xs = xs[np.isfinite(xs)]
    K = (xs.size + 16) // 16 * 16
    amax = np.float32(2.0) ** np.linspace(-30, 60, 64).astype(np.float32)
    amax[0] = np.float32(3e-6)
    rows = np.zeros((64, K), np.float32)
    for m in range(64):
        a = np.float32(amax[m])
        rows[m, 0] = a
        rows[m, 1:1 + xs.size] = np.clip(xs, -a, a)
    rb = workloads.to_bf16_bits(rows)
    say(f"act_quant exhaustive bf16 M=64 K={K}")
    quantized(env, rb, 64, K)


def test_act_quant_scale_sweep(env):
    # s_x = a'/127 and the quantization at inexact 127/a' for every positive
    # finite bf16 absmax: 16 values per row near rounding ties.
    torch, tq, oracle = env
    bits = np.arange(1 << 15, dtype=np.uint32)
    a_all = (bits << 16).view(np.float32)
    a_all = a_all[np.isfinite(a_all) & (a_all > 0)]
    frac = (np.arange(15, dtype=np.float32) + np.float32(0.5)) / np.float32(15.3)
    for c0 in range(0, a_all.size, 64):
        a = a_all[c0:c0 + 64]
        rows = np.zeros((a.size, 16), np.float32)
        rows[:, 0] = a
        rows[:, 1:] = a[:, None] * frac[None, :]
        rb = workloads.to_bf16_bits(rows)
        quantized(env, rb, a.size, 16)


# ------------------------------------------------------------------ gemv
# Covers: 16..256-lane teams, 1..8 pieces per lane with and without a ragged
# last piece, cross-wave team reductions, persistent blocks walking several
# rows, the largest register-path K (32768) and the LDS kernel just above it.
GEMV_SHAPES = [(4, 16), (8, 32), (12, 48), (100, 1008), (36, 2064), (260, 400),
               (2560, 2560), (640, 2560), (6912, 2560), (2560, 6912),
               (4, 131072), (2052, 16), (8, 32768), (4, 32784), (28, 16384),
               (1024, 4608), (40000, 64), (3076, 1552), (28672, 4096)]


def run_gemv(env, N, K, seed, s_w=np.float32(0.02)):
    torch, tq, oracle = env
    codes = workloads.ternary_codes(N, K, seed=seed)
    packed, ref_packed = dev_packed(env, codes)
    xb = workloads.activations_bf16(1, K, seed=seed + 1, outliers=True)
    xq, xs, q_ref, s_ref = quantized(env, xb, 1, K)
    acc = torch.empty(N, dtype=torch.int32, device="cuda")
    y = tq.tq_gemv(packed, s_w, xq, xs, acc=acc)
    torch.cuda.synchronize()
    acc_ref, y32 = oracle.gemv(ref_packed, s_w, q_ref, s_ref, N)
    y64 = oracle.rescale(acc_ref, s_w, s_ref, exact=True)
    np.testing.assert_array_equal(acc.cpu().numpy(), acc_ref[0])
    check_y(y.cpu().numpy(), y32[0], y64[0])
    return packed, xq, xs, y


@pytest.mark.parametrize("N,K", GEMV_SHAPES)
def test_gemv(env, N, K):
    say(f"gemv N={N} K={K}")
    run_gemv(env, N, K, seed=N * 3 + K)


@pytest.mark.parametrize("name", ["70b_up", "70b_down", "8b_up", "8b_down"])
def test_gemv_large(env, name):
    N, K = workloads.LARGE_SHAPES[name]
    say(f"gemv {name} N={N} K={K}")
    run_gemv(env, N, K, seed=workloads.seed_for(4, list(workloads.LARGE_SHAPES).index(name)))


def test_gemv_deterministic_and_scales(env):
    torch, tq, oracle = env
    packed, xq, xs, y = run_gemv(env, 2560, 2560, seed=5, s_w=np.float32(-0.75))
    y2 = tq.tq_gemv(packed, np.float32(-0.75), xq, xs)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(y.cpu().numpy().view(np.uint32),
                                  y2.cpu().numpy().view(np.uint32))


def test_gemv_zero_k_and_empty(env):
    torch, tq, _ = env
    packed = torch.empty(4, 0, dtype=torch.uint8, device="cuda")
    xq = torch.empty(0, dtype=torch.int8, device="cuda")
    xs = torch.ones(1, dtype=torch.float32, device="cuda")
    y = torch.full((16,), 7.0, device="cuda")
    acc = torch.full((16,), 7, dtype=torch.int32, device="cuda")
    tq.tq_gemv(packed, 0.5, xq, xs, y, acc)
    torch.cuda.synchronize()
    assert not y.any() and not acc.any()
    packed = torch.empty(0, 64, dtype=torch.uint8, device="cuda")
    tq.tq_gemv(packed, 0.5, torch.zeros(64, dtype=torch.int8, device="cuda"), xs)


# ------------------------------------------------------------------ gate/up
@pytest.mark.parametrize("M,N,K", [(1, 6912, 2560), (1, 20, 48), (1, 100, 1008),
                                   (1, 256, 28672), (1, 8, 40000), (1, 1028, 4608),
                                   (4, 6912, 2560), (17, 68, 80), (64, 6912, 2560),
                                   (16, 2052, 112), (33, 260, 400), (64, 2560, 6912),
                                   (32, 6912, 2560), (32, 2560, 6912), (8, 516, 20000),
                                   (2, 100, 1008), (3, 12, 131072), (1, 28672, 4096),
                                   (48, 6912, 2560), (64, 6916, 2560)])
def test_gate_up_relu2(env, M, N, K):
    torch, tq, oracle = env
    say(f"gate_up M={M} N={N} K={K}")
    cg = workloads.ternary_codes(N, K, seed=4 + N)
    cu = workloads.ternary_codes(N, K, seed=5 + N)
    pg, rg = dev_packed(env, cg)
    pu, ru = dev_packed(env, cu)
    xb = workloads.activations_bf16(M, K, seed=K + M, outliers=True)
    xq, xs, q_ref, s_ref = quantized(env, xb, M, K)
    s_g, s_u = workloads.tensor_scale(4), workloads.tensor_scale(5)
    acc_g = torch.empty(M, N, dtype=torch.int32, device="cuda")
    acc_u = torch.empty(M, N, dtype=torch.int32, device="cuda")
    h = tq.tq_gate_up_relu2(pg, s_g, pu, s_u, xq, xs, acc_gate=acc_g, acc_up=acc_u)
    torch.cuda.synchronize()
    ag, au, h32 = oracle.gate_up_relu2(rg, s_g, ru, s_u, q_ref, s_ref, N)
    _, _, h64 = oracle.gate_up_relu2(rg, s_g, ru, s_u, q_ref, s_ref, N, exact=True)
    np.testing.assert_array_equal(acc_g.cpu().numpy(), ag)
    np.testing.assert_array_equal(acc_u.cpu().numpy(), au)
    hg = h.cpu().numpy().astype(np.float64)
    np.testing.assert_array_equal(h.cpu().numpy().view(np.uint32), h32.view(np.uint32))
    assert np.all(np.abs(hg - h64) <= REL_TOL * np.abs(h64))


# ------------------------------------------------------------------ gemm small
# M = 2 runs on the vector ALU (K <= 16384), M >= 3 on the matrix cores.
# The matrix-core plans these shapes take (quads per block RG, one 256-byte
# group per wave and pass, waves W, passes over K): every RG in
# {1, 2, 3, 4, 8} (3 at M = 64, N = 2560, with K a multiple of 256 and not),
# W 1..16, blocks of up to 8 and up to 16 waves, one to 32 passes, ragged K
# (not a multiple of 256) and ragged N (not a multiple of 16 RG).
GEMM_CASES = [(m, 6912, 2560) for m in (2, 3, 4, 8, 16, 32, 64)] + \
             [(m, 2560, 6912) for m in (2, 3, 4, 16, 32, 64)] + \
             [(3, 20, 48), (5, 68, 80), (17, 260, 400), (33, 100, 1008),
              (63, 64, 16), (48, 2052, 112),
              (2, 20, 16), (3, 52, 4112), (4, 100, 16384), (4, 64, 16400),
              (2, 36, 1040), (4, 8, 32768), (16, 512, 28672), (2, 12, 20000),
              (2, 36, 12288), (3, 8, 131072), (64, 2560, 6928)]


@pytest.mark.parametrize("M,N,K", GEMM_CASES)
def test_gemm_small(env, M, N, K):
    torch, tq, oracle = env
    say(f"gemm_small M={M} N={N} K={K}")
    codes = workloads.ternary_codes(N, K, seed=M + N + K)
    packed, ref = dev_packed(env, codes)
    xb = workloads.activations_bf16(M, K, seed=M * 11 + K, outliers=True)
    xq, xs, q_ref, s_ref = quantized(env, xb, M, K)
    acc = torch.empty(M, N, dtype=torch.int32, device="cuda")
    s_w = workloads.tensor_scale(6)
    y = tq.tq_gemm_small(packed, s_w, xq, xs, acc=acc)
    torch.cuda.synchronize()
    acc_ref, y32 = oracle.gemv(ref, s_w, q_ref, s_ref, N)
    y64 = oracle.rescale(acc_ref, s_w, s_ref, exact=True)
    np.testing.assert_array_equal(acc.cpu().numpy(), acc_ref)
    check_y(y.cpu().numpy(), y32, y64)
    # Row m of the batch equals the M = 1 GEMV of row m, bit for bit.
    for m in (0, M - 1):
        ym = tq.tq_gemv(packed, s_w, xq[m].contiguous(), xs[m:m + 1].contiguous())
        torch.cuda.synchronize()
        np.testing.assert_array_equal(ym.cpu().numpy().view(np.uint32),
                                      y[m].cpu().numpy().view(np.uint32))


def test_gemm_small_zero_k(env):
    torch, tq, _ = env
    packed = torch.empty(8, 0, dtype=torch.uint8, device="cuda")
    xq = torch.empty(5, 0, dtype=torch.int8, device="cuda")
    xs = torch.ones(5, dtype=torch.float32, device="cuda")
    y = tq.tq_gemm_small(packed, 0.5, xq, xs)
    torch.cuda.synchronize()
    assert y.shape == (5, 32) and not y.any()


# ------------------------------------------------------------------ fused
# (8192, 28672) and (8400, 20000) take the rows-by-dispatch-round mapping of
# the bf16 form on a 256-CU part (the second: rounds of unequal row counts,
# pieces past the row end).  (32776, 16400): the fp32 row's two 256-lane
# teams per block walk up to 9 rows each, so their per-row sum slots are
# reused (more than 8 rows) across the periodic barrier.  (8192, 30720): the
# fp32 form's persistent grid is capped at the one block per CU its
# registers allow.  (28672, 4096): a persistent grid of 4 blocks per CU
# (short rows).
FUSED_SHAPES = [(4, 16), (12, 48), (100, 1008), (36, 2064), (2560, 2560),
                (6912, 2560), (2560, 6912), (8, 32768), (4, 32784), (28, 16384),
                (28672, 8192), (8192, 28672), (8400, 20000), (14336, 4096),
                (32776, 16400), (8192, 30720), (28672, 4096)]


@pytest.mark.parametrize("N,K", FUSED_SHAPES)
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_quant_gemv(env, N, K, dtype):
    torch, tq, oracle = env
    say(f"quant_gemv {dtype} N={N} K={K}")
    codes = workloads.ternary_codes(N, K, seed=N * 5 + K)
    packed, ref = dev_packed(env, codes)
    if dtype == "bf16":
        xh = workloads.activations_bf16(1, K, seed=K + 3, outliers=True)
        x = torch.from_numpy(xh.view(np.int16)).view(torch.bfloat16).cuda()[0]
    else:
        xh = workloads.normal_f32(1, K, seed=K + 4, outliers=True) * np.float32(0.3)
        x = torch.from_numpy(xh).cuda()[0]
    s_w = np.float32(0.021)
    acc = torch.empty(N, dtype=torch.int32, device="cuda")
    xq = torch.empty(K, dtype=torch.int8, device="cuda")
    xs = torch.empty(1, dtype=torch.float32, device="cuda")
    y = tq.tq_quant_gemv(x, packed, s_w, acc=acc, xq=xq, x_scale=xs)
    torch.cuda.synchronize()
    q_ref, s_ref = oracle.act_quant(xh.reshape(1, K), dtype)
    np.testing.assert_array_equal(xq.cpu().numpy(), q_ref[0])
    np.testing.assert_array_equal(xs.cpu().numpy().view(np.uint32), s_ref.view(np.uint32))
    acc_ref, y32 = oracle.gemv(ref, s_w, q_ref, s_ref, N)
    np.testing.assert_array_equal(acc.cpu().numpy(), acc_ref[0])
    check_y(y.cpu().numpy(), y32[0], oracle.rescale(acc_ref, s_w, s_ref, exact=True)[0])
    # with the rescale override (the decode chain's unit activation scale)
    unit = torch.tensor([np.float32(1) / np.float32(127)], device="cuda")
    y2 = tq.tq_quant_gemv(x, packed, s_w, xq=xq, x_scale=xs, y_scale=unit)
    torch.cuda.synchronize()
    u = unit.cpu().numpy()
    _, y32u = oracle.gemv(ref, s_w, q_ref, u, N)
    check_y(y2.cpu().numpy(), y32u[0], oracle.rescale(acc_ref, s_w, u, exact=True)[0])


GROUP_CASES = [((2560, 640, 640), 2560, "bf16"),      # 2B-4T q, k, v
               ((20, 0, 36, 100), 1008, "f32"),       # ragged, an empty matrix
               ((8, 12, 4, 16), 28672, "bf16"),       # 256-lane teams
               ((4, 8), 40000, "f32"),                # K > 32768: fallback
               ((12, 4), 0, "bf16"),                  # K == 0
               ((1024,), 4608, "bf16"),
               ((4096, 2048, 2048), 20480, "bf16"),  # rows by dispatch round
               ((8192, 1024, 1024), 8192, "bf16")]   # 70B-class q, k, v


@pytest.mark.parametrize("Ns,K,dtype", GROUP_CASES)
def test_quant_gemv_group(env, Ns, K, dtype):
    torch, tq, oracle = env
    say(f"quant_gemv_group {dtype} Ns={Ns} K={K}")
    packs, refs = [], []
    for i, N in enumerate(Ns):
        codes = workloads.ternary_codes(N, K, seed=31 + 7 * i + N + K)
        if N * K:
            p, r = dev_packed(env, codes)
        else:   # empty: nothing to pack on the device
            p = torch.empty(N // 4, K, dtype=torch.uint8, device="cuda")
            r = oracle.pack(codes)
        packs.append(p)
        refs.append(r)
    scales = [workloads.tensor_scale(i) for i in range(len(Ns))]
    if dtype == "bf16":
        xh = workloads.activations_bf16(1, K, seed=K + 5, outliers=True)
        x = torch.from_numpy(xh.view(np.int16)).view(torch.bfloat16).cuda()[0]
    else:
        xh = workloads.normal_f32(1, K, seed=K + 6, outliers=True)
        x = torch.from_numpy(xh).cuda()[0]
    accs = [torch.full((N,), 7, dtype=torch.int32, device="cuda") for N in Ns]
    xq = torch.empty(K, dtype=torch.int8, device="cuda")
    xs = torch.empty(1, dtype=torch.float32, device="cuda")
    unit = torch.tensor([np.float32(1) / np.float32(127)], device="cuda")
    ys = tq.tq_quant_gemv_group(x, packs, scales, acc=accs, xq=xq, x_scale=xs)
    ysu = tq.tq_quant_gemv_group(x, packs, scales, y_scale=unit)
    torch.cuda.synchronize()
    q_ref, s_ref = oracle.act_quant(xh.reshape(1, K), dtype)
    np.testing.assert_array_equal(xq.cpu().numpy(), q_ref[0])
    np.testing.assert_array_equal(xs.cpu().numpy().view(np.uint32), s_ref.view(np.uint32))
    u = unit.cpu().numpy()
    for i, N in enumerate(Ns):
        acc_ref, y32 = oracle.gemv(refs[i], scales[i], q_ref, s_ref, N)
        np.testing.assert_array_equal(accs[i].cpu().numpy(), acc_ref[0], err_msg=f"acc {i}")
        check_y(ys[i].cpu().numpy(), y32[0],
                oracle.rescale(acc_ref, scales[i], s_ref, exact=True)[0])
        _, y32u = oracle.gemv(refs[i], scales[i], q_ref, u, N)
        check_y(ysu[i].cpu().numpy(), y32u[0],
                oracle.rescale(acc_ref, scales[i], u, exact=True)[0])
        # bit-identical to the single-matrix call
        if N:
            y1 = tq.tq_quant_gemv(x, packs[i], scales[i], y_scale=unit)
            torch.cuda.synchronize()
            np.testing.assert_array_equal(y1.cpu().numpy().view(np.uint32),
                                          ysu[i].cpu().numpy().view(np.uint32))


# (16400, 20480): two 256-lane teams per block walk up to 9 rows of both
# matrices, reusing their per-row sum slots across the periodic barrier.
# (28672, 4096): a persistent grid of 3 blocks per CU (short rows).
@pytest.mark.parametrize("N,K", [(6912, 2560), (20, 48), (1028, 4608), (256, 28672),
                                 (8, 40000), (16400, 20480), (28672, 4096)])
def test_quant_gate_up_relu2(env, N, K):
    torch, tq, oracle = env
    say(f"quant_gate_up N={N} K={K}")
    pg, rg = dev_packed(env, workloads.ternary_codes(N, K, seed=11 + N))
    pu, ru = dev_packed(env, workloads.ternary_codes(N, K, seed=12 + N))
    xh = workloads.normal_f32(1, K, seed=K + 13, outliers=True)
    x = torch.from_numpy(xh).cuda()[0]
    s_g, s_u = workloads.tensor_scale(4), workloads.tensor_scale(5)
    ag = torch.empty(N, dtype=torch.int32, device="cuda")
    au = torch.empty(N, dtype=torch.int32, device="cuda")
    xq = torch.empty(K, dtype=torch.int8, device="cuda")
    xs = torch.empty(1, dtype=torch.float32, device="cuda")
    h = tq.tq_quant_gate_up_relu2(x, pg, s_g, pu, s_u, acc_gate=ag, acc_up=au,
                                  xq=xq, x_scale=xs)
    torch.cuda.synchronize()
    q_ref, s_ref = oracle.act_quant(xh, "f32")
    np.testing.assert_array_equal(xq.cpu().numpy(), q_ref[0])
    g_ref, u_ref, h32 = oracle.gate_up_relu2(rg, s_g, ru, s_u, q_ref, s_ref, N)
    np.testing.assert_array_equal(ag.cpu().numpy(), g_ref[0])
    np.testing.assert_array_equal(au.cpu().numpy(), u_ref[0])
    np.testing.assert_array_equal(h.cpu().numpy().view(np.uint32), h32[0].view(np.uint32))


def test_quant_gemv_edges(env):
    torch, tq, oracle = env
    xq = torch.empty(64, dtype=torch.int8, device="cuda")
    xs = torch.empty(1, dtype=torch.float32, device="cuda")
    xh = workloads.activations_bf16(1, 64, seed=1)
    x = torch.from_numpy(xh.view(np.int16)).view(torch.bfloat16).cuda()[0]
    # N == 0: only the quantized row and its scale are produced
    tq.tq_quant_gemv(x, torch.empty(0, 64, dtype=torch.uint8, device="cuda"), 0.5,
                     xq=xq, x_scale=xs)
    torch.cuda.synchronize()
    q_ref, s_ref = oracle.act_quant(xh, "bf16")
    np.testing.assert_array_equal(xq.cpu().numpy(), q_ref[0])
    # K == 0: y = 0, s_x = 1e-5/127
    e = torch.empty(0, dtype=torch.bfloat16, device="cuda")
    y = tq.tq_quant_gemv(e, torch.empty(4, 0, dtype=torch.uint8, device="cuda"), 0.5,
                         xq=torch.empty(0, dtype=torch.int8, device="cuda"), x_scale=xs)
    torch.cuda.synchronize()
    assert not y.any()
    assert xs.cpu().numpy()[0] == np.float32(np.float32(1e-5) / np.float32(127))


def test_gate_up_zero_k_without_up_matrix(env):
    """K == 0 with no up matrix at all (a null pointer is allowed when there
    is nothing to read): h = +0, for M = 1 and M > 1 and the fused form."""
    torch, tq, _ = env
    import ctypes
    say("gate_up K=0, packed_up NULL")
    lib = tq.lib
    for M in (1, 5):
        h = torch.full((M, 8), 7.0, device="cuda")
        xs = torch.ones(M, dtype=torch.float32, device="cuda")
        st = lib.tq_gate_up_relu2(None, 0.5, None, 0.25, None, ctypes.c_void_p(xs.data_ptr()),
                                  M, 8, 0, ctypes.c_void_p(h.data_ptr()), None, None, None)
        torch.cuda.synchronize()
        assert st == 0
        assert not h.cpu().numpy().view(np.uint32).any()
    h = torch.full((8,), 7.0, device="cuda")
    xs = torch.empty(1, dtype=torch.float32, device="cuda")
    st = lib.tq_quant_gate_up_relu2(None, 0, None, 0.5, None, 0.25, 8, 0,
                                    ctypes.c_void_p(h.data_ptr()), None, None, None,
                                    ctypes.c_void_p(xs.data_ptr()), None, None)
    torch.cuda.synchronize()
    assert st == 0
    assert not h.cpu().numpy().view(np.uint32).any()
    assert xs.item() == np.float32(np.float32(1e-5) / np.float32(127))
