"""GPU parity past 4 GiB of packed weights.

The C ABI accepts up to 2^31 - 1 packed rows of up to 131072 bytes, so byte
offsets into one weight matrix can pass 2^31 and 2^32.  These cases put the
packed rows a kernel reads on both sides of those offsets and compare the
outputs of sampled rows (first, middle, the rows that straddle 2^31 and 2^32
bytes, last) against the CPU oracle: int32 sums bit-exact, fp32 outputs
bit-exact against the oracle's fixed-order rescale.

The matrices (4.3 GB each) are filled on the GPU with random valid packed
bytes: the byte values come from the oracle's own packing of every
combination of codes, drawn uniformly.  The oracle then sees only the
sampled packed rows, as a small packed matrix: packed row i of the planar
layout holds output rows j * (N/4) + i (j = 0..3; j * ceil(N/5) + i for
five weights per byte), so sub-matrix row s stands for those of S[s].
"""
import itertools
import sys

import numpy as np
import pytest

import workloads

pytestmark = pytest.mark.gpu

K_REG = 16384                       # register-resident GEMV and the MFMA GEMM
N4_BIG = (1 << 32) // K_REG + 64    # 262208 packed rows: 4,296,015,872 bytes
K_LONG = 65536                      # the LDS-staged GEMV (K > 32768)
N4_LONG = (1 << 32) // K_LONG + 64  # 65600 packed rows: 4,299,161,600 bytes
N4_GATE = (1 << 31) // K_REG + 32   # 131104 rows per matrix: past 2^31 each


@pytest.fixture(scope="module")
def env():
    import torch
    import bit_gemv_tq_amd as tq
    import oracle
    return torch, tq, oracle


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def sample_rows(n_rows, K):
    """Packed rows around byte offsets 2^31 and 2^32, plus the ends."""
    s = {0, 1, n_rows // 2, n_rows - 2, n_rows - 1}
    for off in (1 << 31, 1 << 32):
        r = off // K
        s |= {r - 1, r, r + 1}
    return np.array(sorted(x for x in s if 0 <= x < n_rows), np.int64)


def valid_bytes(oracle, per_byte):
    """Every packed byte value the oracle produces (81 or 243 of them)."""
    combos = np.array(list(itertools.product((-1, 0, 1), repeat=per_byte)),
                      np.int8).T.copy()  # [per_byte, combos]: one column each
    if per_byte == 4:
        b = oracle.pack(combos)
    else:
        b = oracle.pack3(combos)
    assert b.shape == (1, combos.shape[1])
    vals = np.unique(b[0])
    assert vals.size == combos.shape[1]
    return vals


def random_packed(env, rows, K, lut, seed):
    """[rows, K] uint8 on the GPU, each byte drawn uniformly from lut."""
    torch, _, _ = env
    out = torch.empty(rows, K, dtype=torch.uint8, device="cuda")
    lut_d = torch.from_numpy(lut.astype(np.uint8)).cuda()
    g = torch.Generator(device="cuda").manual_seed(seed)
    step = max(1, (32 << 20) // K)
    for r0 in range(0, rows, step):
        r1 = min(rows, r0 + step)
        idx = torch.randint(0, lut.size, (r1 - r0, K), generator=g, device="cuda")
        out[r0:r1] = lut_d[idx]
    return out


def quantized_rows(env, M, K, seed):
    torch, tq, oracle = env
    xb = workloads.activations_bf16(M, K, seed=seed, outliers=True)
    x = torch.from_numpy(xb.view(np.int16)).view(torch.bfloat16).cuda().reshape(M, K)
    xq, xs = tq.tq_act_quant(x)
    q_ref, s_ref = oracle.act_quant(xb.reshape(M, K), "bf16")
    np.testing.assert_array_equal(xq.cpu().numpy(), q_ref)
    np.testing.assert_array_equal(xs.cpu().numpy().view(np.uint32), s_ref.view(np.uint32))
    return x, xq, xs, q_ref, s_ref


def out_index(rows, n_rows, per_byte):
    """Output rows of packed rows `rows`, in the oracle sub-matrix's order."""
    return np.concatenate([j * n_rows + rows for j in range(per_byte)])


def check(acc_gpu, y_gpu, acc_ref, y_ref):
    np.testing.assert_array_equal(acc_gpu, acc_ref)
    np.testing.assert_array_equal(y_gpu.view(np.uint32), y_ref.view(np.uint32))


def free(torch):
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def test_two_bit_past_4gib(env):
    """tq_gemv, tq_quant_gemv (bf16 row), tq_quant_gemv_group,
    tq_rmsnorm_quant_gemv and tq_gemm_small (M = 4, matrix cores) on one
    4.3 GB matrix, K = 16384."""
    torch, tq, oracle = env
    n4, K = N4_BIG, K_REG
    N = 4 * n4
    say(f"two-bit past 4 GiB: packed [{n4}, {K}] = {n4 * K} bytes")
    packed = random_packed(env, n4, K, valid_bytes(oracle, 4), seed=41)
    rows = sample_rows(n4, K)
    sub = packed[torch.from_numpy(rows).cuda()].cpu().numpy()
    idx = out_index(rows, n4, 4)
    s_w = np.float32(0.021)

    x, xq, xs, q_ref, s_ref = quantized_rows(env, 4, K, seed=43)
    acc_ref = oracle.ternary_matmul(sub, q_ref, 4 * rows.size)
    y_ref = oracle.rescale(acc_ref, s_w, s_ref)

    say("  tq_gemv")
    acc = torch.empty(N, dtype=torch.int32, device="cuda")
    y = tq.tq_gemv(packed, s_w, xq[0], xs[:1], acc=acc)
    torch.cuda.synchronize()
    check(acc.cpu().numpy()[idx], y.cpu().numpy()[idx], acc_ref[0], y_ref[0])

    say("  tq_quant_gemv (bf16 row)")
    acc.fill_(7)
    y = tq.tq_quant_gemv(x[0], packed, s_w, acc=acc)
    torch.cuda.synchronize()
    check(acc.cpu().numpy()[idx], y.cpu().numpy()[idx], acc_ref[0], y_ref[0])
    del y

    say("  tq_quant_gemv_group (a small matrix, then the big one)")
    small = random_packed(env, 64, K, valid_bytes(oracle, 4), seed=42)
    ys = [torch.empty(256, device="cuda"), torch.empty(N, device="cuda")]
    accs = [torch.full((256,), 7, dtype=torch.int32, device="cuda"), acc]
    tq.tq_quant_gemv_group(x[0], [small, packed], [np.float32(0.5), s_w], y=ys, acc=accs)
    torch.cuda.synchronize()
    acc_s = oracle.ternary_matmul(small.cpu().numpy(), q_ref[:1], 256)
    check(accs[0].cpu().numpy(), ys[0].cpu().numpy(), acc_s[0],
          oracle.rescale(acc_s, np.float32(0.5), s_ref[:1])[0])
    check(acc.cpu().numpy()[idx], ys[1].cpu().numpy()[idx], acc_ref[0], y_ref[0])
    del small, ys, accs

    say("  tq_rmsnorm_quant_gemv (bf16 row)")
    rng = np.random.default_rng(44)
    gamma = (1.0 + 0.25 * rng.standard_normal(K)).astype(np.float32)
    gbits = (gamma.view(np.uint32) >> 16).astype(np.uint16)
    xbits = x[0].cpu().view(torch.int16).numpy().view(np.uint16)
    q_r, s_r = oracle.rmsnorm_act_quant(xbits.reshape(1, K), gbits, 1e-5, "bf16")
    xq_r = torch.empty(K, dtype=torch.int8, device="cuda")
    xs_r = torch.empty(1, dtype=torch.float32, device="cuda")
    acc.fill_(7)
    y = tq.tq_rmsnorm_quant_gemv(x[0], torch.from_numpy(gbits.view(np.int16)).view(torch.bfloat16).cuda(),
                                 packed, s_w, eps=1e-5, acc=acc, xq=xq_r, x_scale=xs_r)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(xq_r.cpu().numpy(), q_r[0])
    s_gpu = xs_r.cpu().numpy()
    assert abs(float(s_gpu[0]) - float(s_r[0])) <= np.spacing(s_r[0])  # one ulp
    acc_r = oracle.ternary_matmul(sub, q_r, 4 * rows.size)[0]
    np.testing.assert_array_equal(acc.cpu().numpy()[idx], acc_r)
    # y is the fixed-order fp32 rescale with the scale the call produced
    y_r = oracle.rescale(acc_r, s_w, s_gpu)[0]
    np.testing.assert_array_equal(y.cpu().numpy()[idx].view(np.uint32), y_r.view(np.uint32))
    del acc, y

    say("  tq_gemm_small M = 4")
    acc4 = torch.empty(4, N, dtype=torch.int32, device="cuda")
    y4 = tq.tq_gemm_small(packed, s_w, xq, xs, acc=acc4)
    torch.cuda.synchronize()
    check(acc4.cpu().numpy()[:, idx], y4.cpu().numpy()[:, idx], acc_ref, y_ref)
    del packed, acc4, y4
    free(torch)


def test_two_bit_long_rows_past_4gib(env):
    """tq_gemv with K = 65536 (activations in LDS) on a 4.3 GB matrix."""
    torch, tq, oracle = env
    n4, K = N4_LONG, K_LONG
    say(f"two-bit long rows past 4 GiB: packed [{n4}, {K}] = {n4 * K} bytes")
    packed = random_packed(env, n4, K, valid_bytes(oracle, 4), seed=47)
    rows = sample_rows(n4, K)
    sub = packed[torch.from_numpy(rows).cuda()].cpu().numpy()
    idx = out_index(rows, n4, 4)
    s_w = np.float32(0.017)
    _, xq, xs, q_ref, s_ref = quantized_rows(env, 1, K, seed=53)
    acc_ref = oracle.ternary_matmul(sub, q_ref, 4 * rows.size)
    y_ref = oracle.rescale(acc_ref, s_w, s_ref)
    acc = torch.empty(4 * n4, dtype=torch.int32, device="cuda")
    y = tq.tq_gemv(packed, s_w, xq[0], xs, acc=acc)
    torch.cuda.synchronize()
    check(acc.cpu().numpy()[idx], y.cpu().numpy()[idx], acc_ref[0], y_ref[0])
    del packed, acc, y
    free(torch)


def test_gate_up_past_2gib_each(env):
    """tq_gate_up_relu2 at M = 1 and M = 4 with two 2.1 GB matrices."""
    torch, tq, oracle = env
    n4, K = N4_GATE, K_REG
    N = 4 * n4
    say(f"gate/up past 2 GiB each: 2 x packed [{n4}, {K}] = {n4 * K} bytes")
    lut = valid_bytes(oracle, 4)
    pg = random_packed(env, n4, K, lut, seed=59)
    pu = random_packed(env, n4, K, lut, seed=61)
    rows = sample_rows(n4, K)
    rows_d = torch.from_numpy(rows).cuda()
    sub_g, sub_u = pg[rows_d].cpu().numpy(), pu[rows_d].cpu().numpy()
    idx = out_index(rows, n4, 4)
    s_g, s_u = np.float32(0.023), np.float32(0.029)
    _, xq, xs, q_ref, s_ref = quantized_rows(env, 4, K, seed=67)
    ag, au, h_ref = oracle.gate_up_relu2(sub_g, s_g, sub_u, s_u, q_ref, s_ref, 4 * rows.size)
    for M in (1, 4):
        say(f"  tq_gate_up_relu2 M = {M}")
        acc_g = torch.empty(M, N, dtype=torch.int32, device="cuda")
        acc_u = torch.empty(M, N, dtype=torch.int32, device="cuda")
        h = tq.tq_gate_up_relu2(pg, s_g, pu, s_u, xq[:M], xs[:M],
                                acc_gate=acc_g, acc_up=acc_u)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(acc_g.cpu().numpy()[:, idx], ag[:M])
        np.testing.assert_array_equal(acc_u.cpu().numpy()[:, idx], au[:M])
        np.testing.assert_array_equal(h.reshape(M, N).cpu().numpy()[:, idx].view(np.uint32),
                                      h_ref[:M].view(np.uint32))
        del acc_g, acc_u, h
    del pg, pu
    free(torch)


def test_five_per_byte_past_4gib(env):
    """tq_gemv3 on a 4.3 GB five-per-byte matrix, K = 16384."""
    torch, tq, oracle = env
    n5, K = N4_BIG, K_REG
    N = 5 * n5
    say(f"five per byte past 4 GiB: packed [{n5}, {K}] = {n5 * K} bytes")
    packed = random_packed(env, n5, K, valid_bytes(oracle, 5), seed=71)
    rows = sample_rows(n5, K)
    sub = packed[torch.from_numpy(rows).cuda()].cpu().numpy()
    idx = out_index(rows, n5, 5)
    codes = oracle.unpack3(sub, 5 * rows.size)  # [5 * len(rows), K]
    s_w = np.float32(0.019)
    _, xq, xs, q_ref, s_ref = quantized_rows(env, 1, K, seed=73)
    # exact integer sums of the sampled rows (codes and q are small ints)
    acc_ref = (codes.astype(np.int64) @ q_ref[0].astype(np.int64)).astype(np.int32)
    y_ref = oracle.rescale(acc_ref, s_w, s_ref)[0]
    acc = torch.empty(N, dtype=torch.int32, device="cuda")
    y = tq.tq_gemv3(packed, s_w, xq[0], xs, N, acc=acc)
    torch.cuda.synchronize()
    check(acc.cpu().numpy()[idx], y.cpu().numpy()[idx], acc_ref, y_ref)
    del packed, acc, y
    free(torch)


def test_attention_past_4gib(env):
    """tq_attn_decode over a KV cache of 4.56 GB per tensor: L = 131072
    tokens, 136 KV heads of D = 128 (one query head each), so the rows of
    the last tokens sit past byte offset 2^32.  Sampled heads against the
    fp64 oracle within the attention tests' derived per-element bound."""
    torch, tq, oracle = env
    import test_gpu_attn as ta
    L, Hkv, D = 131072, 136, 128
    H = Hkv
    say(f"attention past 4 GiB: k/v [{L}, {Hkv}, {D}] bf16 = {L * Hkv * D * 2} bytes each")
    g = torch.Generator(device="cuda").manual_seed(79)
    k = torch.empty(L, Hkv, D, dtype=torch.bfloat16, device="cuda")
    v = torch.empty(L, Hkv, D, dtype=torch.bfloat16, device="cuda")
    step = 4096
    for t0 in range(0, L, step):
        k[t0:t0 + step] = torch.randn(step, Hkv, D, generator=g, device="cuda").to(torch.bfloat16)
        v[t0:t0 + step] = torch.randn(step, Hkv, D, generator=g, device="cuda").to(torch.bfloat16)
    q = torch.randn(H, D, generator=g, device="cuda")
    ws = tq.attn_workspace(H, D, L, q.device)
    out = tq.tq_attn_decode(q, k, v, workspace=ws)
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.float64)
    scale = np.float32(1.0 / np.sqrt(D))
    for h in (0, 67, H - 1):
        kh = k[:, h, :].contiguous().cpu().view(torch.int16).numpy().view(np.uint16)[:, None, :]
        vh = v[:, h, :].contiguous().cpu().view(torch.int16).numpy().view(np.uint16)[:, None, :]
        qh = q[h:h + 1].cpu().numpy()
        ref = oracle.attn_decode(qh, kh, vh, scale)
        tol = ta.bound(qh, kh, vh, ref, scale, L, 1, D)
        err = np.abs(got[h:h + 1] - ref)
        assert np.all(err <= tol), (h, float(np.max(err / tol)))
    del k, v, q, ws, out
    free(torch)


@pytest.mark.parametrize("per_byte", [4, 5])
def test_pack_past_4gib(env, per_byte):
    """tq_pack / tq_pack3 writing a 4.3 GB packed matrix (from 17 / 21 GB of
    int8 codes): sampled packed rows equal the oracle's packing of their
    code rows."""
    torch, tq, oracle = env
    n_rows, K = N4_BIG, K_REG
    N = per_byte * n_rows
    say(f"pack ({per_byte} per byte) past 4 GiB: codes [{N}, {K}], packed [{n_rows}, {K}]")
    g = torch.Generator(device="cuda").manual_seed(83 + per_byte)
    w = torch.empty(N, K, dtype=torch.int8, device="cuda")
    step = (256 << 20) // K
    for r0 in range(0, N, step):
        r1 = min(N, r0 + step)
        w[r0:r1] = torch.randint(-1, 2, (r1 - r0, K), generator=g, device="cuda",
                                 dtype=torch.int8)
    packed = tq.tq_pack(w) if per_byte == 4 else tq.tq_pack3(w)
    torch.cuda.synchronize()
    assert packed.shape == (n_rows, K)
    rows = sample_rows(n_rows, K)
    idx = torch.from_numpy(out_index(rows, n_rows, per_byte)).cuda()
    codes = w[idx].cpu().numpy()  # [per_byte * len(rows), K], sub-matrix order
    ref = oracle.pack(codes) if per_byte == 4 else oracle.pack3(codes)
    np.testing.assert_array_equal(packed[torch.from_numpy(rows).cuda()].cpu().numpy(), ref)
    del w, packed
    free(torch)
