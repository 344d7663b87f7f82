"""GPU parity of tq_attn_decode against the float64 oracle, at the 2B-4T
head layout (20 query heads, 5 KV heads, D = 128) for L from 1 to 32768
(ragged chunk tails included), the other group sizes and D = 64, peaked
softmax, exact cases (one token: out == v; identical keys), and bitwise
determinism across calls.

Covered: one chunk (the chunk pass writes the output), the combine over 2
to 64 chunks of one or several steps, both block sizes (4 waves for short
contexts whose chunks fit one block per CU, else 8 waves with the chunk
count capped at CUs / KV heads), both step sizes (contexts up to 8192 take
the smaller), ragged last steps and chunks, and one workspace reused across
calls of different lengths.

Tolerance (derived from the kernel's fp32 arithmetic, per head h):
  E   = gamma(13) * scale * max_t sum_d |q[h,d] k[t,d]|   (score error: an
        8-term FMA chain, a 16-lane tree, the scale product)
  rho = 2E + u * max_t |s_t - m| + 2^-22                 (relative weight
        error: scores, the subtraction, expf within 2 ulp)
  |out - o| <= 2 max|v| rho + gamma(dN) max|v| + gamma(dD) |o| + ulp32(o)
with gamma(n) = n u / (1 - n u), u = 2^-24, dN / dD the summation depths of
the numerator / denominator (tokens per lane, shuffle and wave trees, the
fp64 merge of the splits is exact to well below u).
"""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def env():
    import torch
    import bit_gemv_tq_amd as tq
    import oracle
    return torch, tq, oracle


def make(L, H, Hkv, D, seed, kscale=1.0):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((H, D)).astype(np.float32)
    kf = (rng.standard_normal((L, Hkv, D)) * kscale).astype(np.float32)
    vf = rng.standard_normal((L, Hkv, D)).astype(np.float32)
    tobf = lambda a: (a.view(np.uint32) >> 16).astype(np.uint16)
    return q, tobf(kf), tobf(vf)


def ulp32(x):
    a = np.abs(x).astype(np.float32)
    return (np.nextafter(a, np.float32(np.inf)) - a).astype(np.float64)


U = 2.0 ** -24


def gamma(n):
    return n * U / (1 - n * U)


def num_cus():
    import torch
    return torch.cuda.get_device_properties(0).multi_processor_count


def chunk_shape(G, D, L, Hkv, cus):
    """Tokens per lane slot over a chunk, tokens per chunk and waves per
    block of the kernel's plan (steps of 4 tokens per lane slot, or D/8/G
    where that is more): one 8-wave chunk up to 256 tokens where 4-wave
    steps would need more than one chunk; 4-wave blocks (up to 64 chunks per
    KV head) for contexts up to 8192 whose chunks number at most one block
    per CU;
    otherwise 8-wave blocks with at most CUs / Hkv chunks per KV head (more where a chunk's G score
    rows would pass 128 KiB of LDS).  Whole steps per chunk."""
    lpt = D // 8                                   # lanes per token row
    tpw = 64 // lpt                                # token slots per wave
    kt = max(lpt // G, 4)                          # tokens per slot and step
    if L <= 8192:
        step = 4 * tpw * kt
        steps = -(-L // (step * 64))
        chunks = -(-L // (steps * step))
        if chunks > 1 and L <= 256:                # one chunk of 8-wave steps
            n8 = -(-L // (8 * tpw * kt))
            return n8 * kt, n8 * 8 * tpw * kt, 8
        if Hkv * chunks <= cus:
            return steps * kt, steps * step, 4
    lds_min = -(-L * G * 4 // (128 * 1024))        # scores of a chunk <= 128 KiB
    cap = min(64, max(1, cus // Hkv, lds_min))
    step = 8 * tpw * kt
    steps = -(-L // (step * cap))
    return steps * kt, steps * step, 8


def bound(q, k, v, ref, scale, L, G, D):
    """Per-element error bound of the kernel's fp32 arithmetic (see above)."""
    kf = (k.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    vf = (v.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    kt, chunk, nw = chunk_shape(G, D, L, q.shape[0] // G, num_cus())
    dN = kt + 4 + nw   # a slot's tokens, 3 shuffle levels, the waves
    dD = -(-chunk // (64 * nw)) + 7 + nw
    H = q.shape[0]
    out = np.empty_like(ref)
    for h in range(H):
        g = h // G
        absdot = np.abs(kf[:, g, :]) @ np.abs(q[h].astype(np.float64))
        s = (kf[:, g, :] @ q[h].astype(np.float64)) * float(scale)
        E = gamma(13) * float(scale) * absdot.max()
        rho = 2 * E + U * np.max(s.max() - s) + 2.0 ** -22
        vmax = np.abs(vf[:, g, :]).max()
        out[h] = 2 * vmax * rho + gamma(dN) * vmax + gamma(dD) * np.abs(ref[h]) + ulp32(ref[h])
    return out


def check(env, L, H=20, Hkv=5, D=128, seed=0, kscale=1.0, data=None, ws=None):
    torch, tq, oracle = env
    print(f"attn L={L} H={H} Hkv={Hkv} D={D}", flush=True)
    q, k, v = make(L, H, Hkv, D, seed, kscale) if data is None else data
    qt = torch.from_numpy(q).cuda()
    kt = torch.from_numpy(k.view(np.int16)).view(torch.bfloat16).cuda()
    vt = torch.from_numpy(v.view(np.int16)).view(torch.bfloat16).cuda()
    out = tq.tq_attn_decode(qt, kt, vt, workspace=ws)
    torch.cuda.synchronize()
    scale = np.float32(1.0 / np.sqrt(D))
    ref = oracle.attn_decode(q, k, v, scale)
    got = out.cpu().numpy().astype(np.float64)
    tol = bound(q, k, v, ref, scale, L, H // Hkv, D)
    err = np.abs(got - ref)
    assert np.all(err <= tol), float(np.max(err / tol))
    return qt, kt, vt, out


# here (256 CUs, 5 KV heads): 4-wave blocks of 64-token steps up to L = 3264
# (one chunk up to 64 tokens, 51 chunks at 3264), then 8-wave blocks of
# 128-token steps, at most 51 chunks per KV head (131072: 49 chunks of 21
# steps)
@pytest.mark.parametrize("L", [1, 7, 16, 64, 65, 100, 2048, 2049, 3264, 3265, 4096,
                               8192, 8193, 32768, 131072])
def test_attn_2b4t_heads(env, L):
    check(env, L, seed=L)


@pytest.mark.parametrize("L", [777, 5000])
@pytest.mark.parametrize("H,Hkv,D", [(8, 8, 128), (16, 8, 64), (32, 4, 128), (4, 1, 64),
                                     (64, 8, 128), (16, 2, 64)])
def test_attn_group_sizes(env, H, Hkv, D, L):
    check(env, L, H, Hkv, D, seed=H + D + L)


@pytest.mark.parametrize("H,Hkv,D,L", [(256, 32, 64, 40000), (64, 8, 128, 131072)])
def test_attn_many_kv_heads_long(env, H, Hkv, D, L):
    # many KV heads at long contexts: few chunks per KV head, so the chunk
    # length is bounded by the LDS that holds its scores (256 / 32 heads:
    # 10 chunks of 4096 tokens rather than 8 of 5120)
    check(env, L, H, Hkv, D, seed=H + L)


def test_attn_workspace_reuse(env):
    # one workspace across lengths with different chunk sizes and counts
    torch, tq, _ = env
    ws = tq.attn_workspace(20, 128, 40000, "cuda")
    for i, L in enumerate([5000, 100, 40000, 1, 8193, 300]):
        ws.fill_(0xFF)
        check(env, L, seed=900 + i, ws=ws)


def test_attn_peaked_scores(env):
    # large key scale: softmax concentrated on few tokens (max subtraction)
    check(env, 4096, seed=5, kscale=30.0)


def test_attn_exact_cases(env):
    torch, tq, _ = env
    # one token: weight exactly 1, so out is v (widened) bit for bit
    q, k, v = make(1, 20, 5, 128, 21)
    _, _, _, out = check(env, 1, data=(q, k, v))
    vf = (v.astype(np.uint32) << 16).view(np.float32)
    for h in range(20):
        np.testing.assert_array_equal(out[h].cpu().numpy(), vf[0, h // 4])
    # identical keys: every weight is exactly 1; out is the mean of v
    q, k, v = make(300, 20, 5, 128, 22)
    k[:] = k[0]
    check(env, 300, data=(q, k, v))


def test_attn_deterministic(env):
    torch, tq, _ = env
    qt, kt, vt, out = check(env, 5000, seed=6)
    for _ in range(3):
        again = tq.tq_attn_decode(qt, kt, vt)
        torch.cuda.synchronize()
        assert torch.equal(again.view(torch.int32), out.view(torch.int32))
