"""GPU parity on the method's closed-form cases.

Page "BitNet" (news digest), first item: with weights in {-1,0,1} every
product is an add, a subtract or a skip.  So the exact sums have closed
forms for structured weights, and those structures drive the kernels'
scaled code planes to their extremes, which random weights never do:

  * W = 0           -> acc = 0 and y = +0 (positive scales);
  * W = +1 / -1     -> acc = +-sum_k q_k  (every q = +127: |acc| = 127 K,
                       the largest sum the contract allows at K = 131072);
  * W = +-I (N = K) -> acc = +-q;
  * W = checkerboard (-1)^(n+k)
                    -> acc[n] = (-1)^n sum_k (-1)^k q_k  (with alternating
                       q = +-127 this is again +-127 K).

Every result is compared element by element with the CPU oracle (int32 sums
bit-exact, fp32 outputs bit-exact against its fixed-order rescale and within
1e-6 of its exact value) and, independently, with the closed form computed
here in int64 from the quantized activations.  Kernels covered: the M = 1
GEMV (int8 row and the fused bf16 prologue, both K ranges), the small-batch
GEMM on the vector ALU (M = 2) and the matrix cores (M = 3..64: the 64 (c-2)
plane-3 decode reaches -128 * 127 * K there), the gate/up + relu^2 projection
at M = 1 and M > 1, and the five-per-byte GEMV.  Activations with q = +-127
come from rows of +-1.0 (absmax 1, 127/1 exact); an all-zero row quantizes
to zero codes with s_x = 1e-5/127.
"""
import sys

import numpy as np
import pytest

import workloads

pytestmark = pytest.mark.gpu

REL_TOL = 1e-6
# (K, N): K spans one piece, the 2B-4T hidden size, the register path's
# largest K, the LDS kernel just above it and the contract's largest K; N is
# a ragged multiple of 4 sized so the oracle stays quick.
K_CASES = [(16, 2564), (2560, 1028), (32768, 132), (32784, 68), (131072, 36)]
W_CONST = ("zero", "plus", "minus")
W_SQUARE = ("eye", "neye", "checker")


@pytest.fixture(scope="module")
def env():
    import torch
    import bit_gemv_tq_amd as tq
    import oracle
    return torch, tq, oracle


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def weights(kind, N, K):
    if kind == "zero":
        return np.zeros((N, K), np.int8)
    if kind == "plus":
        return np.ones((N, K), np.int8)
    if kind == "minus":
        return -np.ones((N, K), np.int8)
    assert N == K
    if kind == "eye":
        return np.eye(N, dtype=np.int8)
    if kind == "neye":
        return -np.eye(N, dtype=np.int8)
    if kind == "checker":
        n = np.arange(N)[:, None]
        k = np.arange(K)[None, :]
        return np.where((n + k) % 2 == 0, 1, -1).astype(np.int8)
    raise ValueError(kind)


def closed_form(kind, q):
    """Exact sums [M, N] of the structured weights, from the codes q [M, K]."""
    q = q.astype(np.int64)
    M, K = q.shape
    sign_k = np.where(np.arange(K) % 2 == 0, 1, -1)
    if kind == "zero":
        return np.zeros((M, 1), np.int64)
    if kind == "plus":
        return q.sum(axis=1, keepdims=True)
    if kind == "minus":
        return -q.sum(axis=1, keepdims=True)
    if kind == "eye":
        return q.copy()
    if kind == "neye":
        return -q
    if kind == "checker":
        s = (q * sign_k[None, :]).sum(axis=1, keepdims=True)
        return s * sign_k[None, :]  # (-1)^n with n over N = K
    raise ValueError(kind)


def check_closed(kind, acc, q):
    """acc [M, N] against the closed form (broadcast over N for constants)."""
    want = closed_form(kind, q)
    np.testing.assert_array_equal(acc.astype(np.int64),
                                  np.broadcast_to(want, acc.shape))


def act_rows(kind, M, K):
    """bf16 bit patterns [M, K] whose codes are +-127 (or 0 for zero rows).

    all127: every entry +1.0 (q = +127); alt127: +1, -1, ... (row m starts
    with (-1)^m); mixed: rows cycle through +1.0, -1.0, alternating and
    all-zero."""
    k = np.arange(K)
    rows = np.empty((M, K), np.float32)
    for m in range(M):
        if kind == "all127":
            rows[m] = 1.0
        elif kind == "alt127":
            rows[m] = np.where((k + m) % 2 == 0, 1.0, -1.0)
        elif kind == "mixed":
            c = m % 4
            if c == 2:
                rows[m] = np.where(k % 2 == 0, -1.0, 1.0)
            else:
                rows[m] = (1.0, -1.0, None, 0.0)[c]
        else:
            raise ValueError(kind)
    return workloads.to_bf16_bits(rows)


def dev_bf16(env, bits):
    torch = env[0]
    return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).cuda()


def quantize(env, bits):
    """GPU act-quant of bf16 rows, checked bit-exact against the oracle."""
    torch, tq, oracle = env
    xq, xs = tq.tq_act_quant(dev_bf16(env, bits))
    torch.cuda.synchronize()
    q_ref, s_ref = oracle.act_quant(bits, "bf16")
    np.testing.assert_array_equal(xq.cpu().numpy(), q_ref)
    np.testing.assert_array_equal(xs.cpu().numpy().view(np.uint32),
                                  s_ref.view(np.uint32))
    return xq, xs, q_ref, s_ref


def packed_pair(env, codes):
    torch, tq, oracle = env
    p = tq.tq_pack(torch.from_numpy(codes).cuda())
    ref = oracle.pack(codes)
    np.testing.assert_array_equal(p.cpu().numpy(), ref)
    return p, ref


def check_y(y, y32, y64):
    y = np.asarray(y).reshape(y32.shape)
    np.testing.assert_array_equal(y.view(np.uint32), y32.view(np.uint32))
    err = np.abs(y.astype(np.float64) - y64)
    assert np.all(err <= REL_TOL * np.abs(y64))


def weight_cases(K, N):
    """(kind, N) pairs for one K: the constant patterns at the ragged N, and
    at K = 2560 also the square patterns (N = K)."""
    out = [(w, N) for w in W_CONST]
    if K == 2560:
        out += [(w, K) for w in W_SQUARE]
    return out


# ------------------------------------------------------------------ act quant
def test_act_quant_zero_rows(env):
    """An all-zero row between ordinary rows (M = 4): codes 0, s_x = 1e-5/127."""
    torch, tq, oracle = env
    say("act_quant zero rows M=4 K=2560")
    x = workloads.normal_f32(4, 2560, seed=77, outliers=True)
    x[1] = 0.0
    x[3] = 0.0
    bits = workloads.to_bf16_bits(x)
    xq, xs, q_ref, s_ref = quantize(env, bits)
    assert not xq[1].any() and not xq[3].any()
    floor = np.float32(np.float32(1e-5) / np.float32(127))
    assert xs[1].item() == floor and xs[3].item() == floor
    # the same rows through the matrix-core GEMM: zero rows give y = +0
    codes = workloads.ternary_codes(256, 2560, seed=78)
    p, ref = packed_pair(env, codes)
    acc = torch.empty(4, 256, dtype=torch.int32, device="cuda")
    y = tq.tq_gemm_small(p, np.float32(0.02), xq, xs, acc=acc)
    torch.cuda.synchronize()
    acc_ref, y32 = oracle.gemv(ref, np.float32(0.02), q_ref, s_ref, 256)
    np.testing.assert_array_equal(acc.cpu().numpy(), acc_ref)
    check_y(y.cpu().numpy(), y32, oracle.rescale(acc_ref, np.float32(0.02), s_ref, exact=True))
    yb = y.cpu().numpy().view(np.uint32)
    assert not yb[1].any() and not yb[3].any()   # +0, not -0


# ------------------------------------------------------------------ M = 1
@pytest.mark.parametrize("K,N", K_CASES)
def test_gemv_closed_forms(env, K, N):
    torch, tq, oracle = env
    s_w = np.float32(0.02)
    for akind in ("all127", "alt127"):
        bits = act_rows(akind, 1, K)
        xq, xs, q_ref, s_ref = quantize(env, bits)
        assert np.all(np.abs(q_ref) == 127)
        for wkind, n in weight_cases(K, N):
            say(f"gemv K={K} N={n} W={wkind} x={akind}")
            p, ref = packed_pair(env, weights(wkind, n, K))
            acc = torch.full((n,), 7, dtype=torch.int32, device="cuda")
            y = tq.tq_gemv(p, s_w, xq[0], xs, acc=acc)
            torch.cuda.synchronize()
            acc_ref, y32 = oracle.gemv(ref, s_w, q_ref, s_ref, n)
            got = acc.cpu().numpy()[None, :]
            np.testing.assert_array_equal(got, acc_ref)
            check_closed(wkind, got, q_ref)
            check_y(y.cpu().numpy()[None, :], y32,
                    oracle.rescale(acc_ref, s_w, s_ref, exact=True))
            if wkind == "zero":
                assert not y.cpu().numpy().view(np.uint32).any()  # +0


@pytest.mark.parametrize("K,N", K_CASES)
def test_quant_gemv_closed_forms(env, K, N):
    """The fused bf16 prologue (K > 32768: its two-launch form)."""
    torch, tq, oracle = env
    s_w = np.float32(0.021)
    for akind in ("all127", "alt127"):
        bits = act_rows(akind, 1, K)
        x = dev_bf16(env, bits)[0]
        q_ref, s_ref = oracle.act_quant(bits, "bf16")
        for wkind, n in weight_cases(K, N):
            say(f"quant_gemv K={K} N={n} W={wkind} x={akind}")
            p, ref = packed_pair(env, weights(wkind, n, K))
            acc = torch.full((n,), 7, dtype=torch.int32, device="cuda")
            xq = torch.empty(K, dtype=torch.int8, device="cuda")
            xs = torch.empty(1, dtype=torch.float32, device="cuda")
            y = tq.tq_quant_gemv(x, p, s_w, acc=acc, xq=xq, x_scale=xs)
            torch.cuda.synchronize()
            np.testing.assert_array_equal(xq.cpu().numpy(), q_ref[0])
            np.testing.assert_array_equal(xs.cpu().numpy().view(np.uint32),
                                          s_ref.view(np.uint32))
            acc_ref, y32 = oracle.gemv(ref, s_w, q_ref, s_ref, n)
            got = acc.cpu().numpy()[None, :]
            np.testing.assert_array_equal(got, acc_ref)
            check_closed(wkind, got, q_ref)
            check_y(y.cpu().numpy()[None, :], y32,
                    oracle.rescale(acc_ref, s_w, s_ref, exact=True))


# ------------------------------------------------------------------ M > 1
@pytest.mark.parametrize("M", [2, 3, 4, 16, 64])
@pytest.mark.parametrize("K,N", K_CASES)
def test_gemm_small_closed_forms(env, M, K, N):
    torch, tq, oracle = env
    s_w = np.float32(0.026)
    for akind in ("all127", "alt127", "mixed"):
        bits = act_rows(akind, M, K)
        xq, xs, q_ref, s_ref = quantize(env, bits)
        for wkind, n in weight_cases(K, N):
            say(f"gemm_small M={M} K={K} N={n} W={wkind} x={akind}")
            p, ref = packed_pair(env, weights(wkind, n, K))
            acc = torch.full((M, n), 7, dtype=torch.int32, device="cuda")
            y = tq.tq_gemm_small(p, s_w, xq, xs, acc=acc)
            torch.cuda.synchronize()
            acc_ref, y32 = oracle.gemv(ref, s_w, q_ref, s_ref, n)
            got = acc.cpu().numpy()
            np.testing.assert_array_equal(got, acc_ref)
            check_closed(wkind, got, q_ref)
            check_y(y.cpu().numpy(), y32, oracle.rescale(acc_ref, s_w, s_ref, exact=True))


# ------------------------------------------------------------------ gate/up
GATE_PAIRS = (("plus", "minus"), ("minus", "plus"), ("zero", "plus"),
              ("plus", "zero"))


@pytest.mark.parametrize("M", [1, 4, 64])
@pytest.mark.parametrize("K,N", K_CASES)
def test_gate_up_closed_forms(env, M, K, N):
    torch, tq, oracle = env
    s_g, s_u = workloads.tensor_scale(4), workloads.tensor_scale(5)
    pairs = [(g, u, N) for g, u in GATE_PAIRS]
    if K == 2560:
        pairs += [("checker", "eye", K), ("neye", "checker", K)]
    for akind in ("all127", "alt127") + (("mixed",) if M > 1 else ()):
        bits = act_rows(akind, M, K)
        xq, xs, q_ref, s_ref = quantize(env, bits)
        for gk, uk, n in pairs:
            say(f"gate_up M={M} K={K} N={n} gate={gk} up={uk} x={akind}")
            pg, rg = packed_pair(env, weights(gk, n, K))
            pu, ru = packed_pair(env, weights(uk, n, K))
            ag = torch.full((M, n), 7, dtype=torch.int32, device="cuda")
            au = torch.full((M, n), 7, dtype=torch.int32, device="cuda")
            h = tq.tq_gate_up_relu2(pg, s_g, pu, s_u, xq, xs, acc_gate=ag, acc_up=au)
            torch.cuda.synchronize()
            g_ref, u_ref, h32 = oracle.gate_up_relu2(rg, s_g, ru, s_u, q_ref, s_ref, n)
            _, _, h64 = oracle.gate_up_relu2(rg, s_g, ru, s_u, q_ref, s_ref, n, exact=True)
            np.testing.assert_array_equal(ag.cpu().numpy(), g_ref)
            np.testing.assert_array_equal(au.cpu().numpy(), u_ref)
            check_closed(gk, ag.cpu().numpy(), q_ref)
            check_closed(uk, au.cpu().numpy(), q_ref)
            check_y(h.cpu().numpy(), h32, h64)


@pytest.mark.parametrize("K,N", K_CASES)
def test_quant_gate_up_closed_forms(env, K, N):
    torch, tq, oracle = env
    s_g, s_u = workloads.tensor_scale(4), workloads.tensor_scale(5)
    for akind in ("all127", "alt127"):
        bits = act_rows(akind, 1, K)
        x = dev_bf16(env, bits)[0]
        q_ref, s_ref = oracle.act_quant(bits, "bf16")
        for gk, uk in GATE_PAIRS:
            say(f"quant_gate_up K={K} N={N} gate={gk} up={uk} x={akind}")
            pg, rg = packed_pair(env, weights(gk, N, K))
            pu, ru = packed_pair(env, weights(uk, N, K))
            ag = torch.full((N,), 7, dtype=torch.int32, device="cuda")
            au = torch.full((N,), 7, dtype=torch.int32, device="cuda")
            h = tq.tq_quant_gate_up_relu2(x, pg, s_g, pu, s_u, acc_gate=ag, acc_up=au)
            torch.cuda.synchronize()
            g_ref, u_ref, h32 = oracle.gate_up_relu2(rg, s_g, ru, s_u, q_ref, s_ref, N)
            np.testing.assert_array_equal(ag.cpu().numpy()[None, :], g_ref)
            np.testing.assert_array_equal(au.cpu().numpy()[None, :], u_ref)
            check_closed(gk, ag.cpu().numpy()[None, :], q_ref)
            np.testing.assert_array_equal(h.cpu().numpy()[None, :].view(np.uint32),
                                          h32.view(np.uint32))


# ------------------------------------------------------------------ gemv3
@pytest.mark.parametrize("K,N", [(16, 2563), (2560, 1027), (32768, 131)])
def test_gemv3_closed_forms(env, K, N):
    """Five weights per byte: every byte of a constant pattern is one value
    (W = -1: all digits 0; W = +1: all digits 2), the two ends of the
    base-3 range.  N % 5 != 0, so the padding rows (zero weights) mix in."""
    torch, tq, oracle = env
    s_w = np.float32(0.019)
    cases = [(w, N) for w in W_CONST] + ([(w, K) for w in W_SQUARE] if K == 2560 else [])
    for akind in ("all127", "alt127"):
        bits = act_rows(akind, 1, K)
        xq, xs, q_ref, s_ref = quantize(env, bits)
        for wkind, n in cases:
            say(f"gemv3 K={K} N={n} W={wkind} x={akind}")
            codes = weights(wkind, n, K)
            p3 = tq.tq_pack3(torch.from_numpy(codes).cuda())
            ref_bytes = oracle.pack3(codes)
            np.testing.assert_array_equal(p3.cpu().numpy(), ref_bytes)
            acc = torch.full((n,), 7, dtype=torch.int32, device="cuda")
            y = tq.tq_gemv3(p3, s_w, xq[0], xs, n, acc=acc)
            torch.cuda.synchronize()
            unpacked = oracle.unpack3(ref_bytes, n)
            pad = (-n) % 4
            acc_ref, y32 = oracle.gemv(
                oracle.pack(np.vstack([unpacked, np.zeros((pad, K), np.int8)])),
                s_w, q_ref, s_ref, n + pad)
            got = acc.cpu().numpy()[None, :]
            np.testing.assert_array_equal(got, acc_ref[:, :n])
            check_closed(wkind, got, q_ref)
            np.testing.assert_array_equal(y.cpu().numpy()[None, :].view(np.uint32),
                                          y32[:, :n].view(np.uint32))


# ------------------------------------------------------------------ grouped, RMSNorm
@pytest.mark.parametrize("K", [2560, 32768, 32784])
def test_quant_gemv_group_closed_forms(env, K):
    """Several matrices sharing one activation row (the q/k/v launch), each a
    different structured pattern, in one launch (K > 32768: its fallback)."""
    torch, tq, oracle = env
    kinds = ("plus", "minus", "zero")
    Ns = (36, 20, 12)
    scales = [np.float32(0.02), np.float32(0.021), np.float32(0.022)]
    for akind in ("all127", "alt127"):
        bits = act_rows(akind, 1, K)
        x = dev_bf16(env, bits)[0]
        q_ref, s_ref = oracle.act_quant(bits, "bf16")
        say(f"quant_gemv_group K={K} x={akind}")
        packs, refs = zip(*[packed_pair(env, weights(k, n, K)) for k, n in zip(kinds, Ns)])
        accs = [torch.full((n,), 7, dtype=torch.int32, device="cuda") for n in Ns]
        ys = tq.tq_quant_gemv_group(x, list(packs), scales, acc=accs)
        torch.cuda.synchronize()
        for i, (k, n) in enumerate(zip(kinds, Ns)):
            acc_ref, y32 = oracle.gemv(refs[i], scales[i], q_ref, s_ref, n)
            got = accs[i].cpu().numpy()[None, :]
            np.testing.assert_array_equal(got, acc_ref)
            check_closed(k, got, q_ref)
            check_y(ys[i].cpu().numpy()[None, :], y32,
                    oracle.rescale(acc_ref, scales[i], s_ref, exact=True))


@pytest.mark.parametrize("K", [2560, 32768, 32784])
def test_rmsnorm_quant_gemv_closed_forms(env, K):
    """The RMSNorm-folded prologue with gamma = 1 on rows of +-1: codes
    +-127, so the sums are the closed forms; the scale carries the RMS
    factor (checked against the oracle within one fp32 ulp, as its tests
    allow)."""
    torch, tq, oracle = env
    gbits = workloads.to_bf16_bits(np.ones((1, K), np.float32))[0]
    gamma = dev_bf16(env, gbits)
    s_w = np.float32(0.023)
    for akind in ("all127", "alt127"):
        bits = act_rows(akind, 1, K)
        x = dev_bf16(env, bits)[0]
        q_ref, s_ref = oracle.rmsnorm_act_quant(bits, gbits, 1e-5, "bf16")
        assert np.all(np.abs(q_ref) == 127)
        for wkind in W_CONST:
            say(f"rmsnorm_quant_gemv K={K} W={wkind} x={akind}")
            p, ref = packed_pair(env, weights(wkind, 68, K))
            acc = torch.full((68,), 7, dtype=torch.int32, device="cuda")
            xq = torch.empty(K, dtype=torch.int8, device="cuda")
            xs = torch.empty(1, dtype=torch.float32, device="cuda")
            y = tq.tq_rmsnorm_quant_gemv(x, gamma, p, s_w, eps=1e-5, acc=acc, xq=xq, x_scale=xs)
            torch.cuda.synchronize()
            np.testing.assert_array_equal(xq.cpu().numpy(), q_ref[0])
            sx = xs.cpu().numpy()
            assert abs(int(sx.view(np.int32)[0]) - int(s_ref.view(np.int32)[0])) <= 1
            acc_ref = oracle.ternary_matmul(ref, q_ref, 68)
            got = acc.cpu().numpy()[None, :]
            np.testing.assert_array_equal(got, acc_ref)
            check_closed(wkind, got, q_ref)
            y64 = oracle.rescale(acc_ref, s_w, sx, exact=True)
            err = np.abs(y.cpu().numpy().astype(np.float64) - y64[0])
            assert np.all(err <= REL_TOL * np.abs(y64[0]))


# ------------------------------------------------ widest matrix-core plans
def test_closed_forms_at_the_widest_quad_plans(env):
    """The closed forms through the plans with the most quads per block: the
    small-batch GEMM at M = 64, [2560, 6912] (3 quads per block, 16 waves)
    and the gated pair at M = 64, [6912, 2560] (8 quads of each matrix per
    block), where every plane scale of every quad reaches its extremes."""
    torch, tq, oracle = env
    M = 64
    K, N = 6912, 2560
    s_w = np.float32(0.023)
    for akind in ("all127", "mixed"):
        bits = act_rows(akind, M, K)
        xq, xs, q_ref, s_ref = quantize(env, bits)
        for wkind in ("plus", "minus"):
            say(f"gemm_small widest plan M={M} K={K} N={N} W={wkind} x={akind}")
            p, ref = packed_pair(env, weights(wkind, N, K))
            acc = torch.full((M, N), 7, dtype=torch.int32, device="cuda")
            y = tq.tq_gemm_small(p, s_w, xq, xs, acc=acc)
            torch.cuda.synchronize()
            acc_ref, y32 = oracle.gemv(ref, s_w, q_ref, s_ref, N)
            np.testing.assert_array_equal(acc.cpu().numpy(), acc_ref)
            check_closed(wkind, acc.cpu().numpy(), q_ref)
            check_y(y.cpu().numpy(), y32, oracle.rescale(acc_ref, s_w, s_ref, exact=True))
    K, N = 2560, 6912
    s_g, s_u = workloads.tensor_scale(4), workloads.tensor_scale(5)
    bits = act_rows("mixed", M, K)
    xq, xs, q_ref, s_ref = quantize(env, bits)
    for gk, uk in (("plus", "minus"), ("minus", "plus")):
        say(f"gate_up widest plan M={M} K={K} N={N} gate={gk} up={uk}")
        pg, rg = packed_pair(env, weights(gk, N, K))
        pu, ru = packed_pair(env, weights(uk, N, K))
        ag = torch.full((M, N), 7, dtype=torch.int32, device="cuda")
        au = torch.full((M, N), 7, dtype=torch.int32, device="cuda")
        h = tq.tq_gate_up_relu2(pg, s_g, pu, s_u, xq, xs, acc_gate=ag, acc_up=au)
        torch.cuda.synchronize()
        g_ref, u_ref, h32 = oracle.gate_up_relu2(rg, s_g, ru, s_u, q_ref, s_ref, N)
        _, _, h64 = oracle.gate_up_relu2(rg, s_g, ru, s_u, q_ref, s_ref, N, exact=True)
        np.testing.assert_array_equal(ag.cpu().numpy(), g_ref)
        np.testing.assert_array_equal(au.cpu().numpy(), u_ref)
        check_closed(gk, ag.cpu().numpy(), q_ref)
        check_closed(uk, au.cpu().numpy(), q_ref)
        check_y(h.cpu().numpy(), h32, h64)
