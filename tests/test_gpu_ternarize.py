"""GPU parity of tq_ternarize (absmean ternarization of bf16 weights)
against the oracle: the weight scale bit for bit and the packed codes byte
for byte, on seeded synthetic bf16 weights N(0, 0.02^2) at the 2B-4T and
8B-class shapes, ragged small shapes, a tensor whose mean makes one code an
exact fp32 tie, all-zero and sub-floor tensors, and random bf16 bit
patterns spanning subnormals to the largest finite value.
"""
import numpy as np
import pytest

import workloads
from tests.test_oracle_ternarize import tie_matrix

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def env():
    import torch
    import bit_gemv_tq_amd as tq
    import oracle
    return torch, tq, oracle


def run(env, bits):
    torch, tq, oracle = env
    N, K = bits.shape
    print(f"ternarize N={N} K={K}", flush=True)
    w = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).cuda()
    packed, s = tq.tq_ternarize(w)
    torch.cuda.synchronize()
    codes, s_ref = oracle.ternarize(bits)
    assert s.cpu().numpy().view(np.uint32)[0] == np.float32(s_ref).view(np.uint32), \
        (float(s.cpu()[0]), float(s_ref))
    np.testing.assert_array_equal(packed.cpu().numpy(), oracle.pack(codes))
    return codes, s_ref


@pytest.mark.parametrize("N,K", [(4, 16), (8, 48), (20, 1008), (2560, 2560),
                                 (6912, 2560), (2560, 6912), (14336, 4096)])
def test_ternarize_gaussian(env, N, K):
    codes, s = run(env, workloads.weights_bf16(N, K, seed=N + K))
    if N * K >= 1 << 20:   # sanity of the statistic on large tensors
        assert abs(float(s) - 0.02 * np.sqrt(2 / np.pi)) < 2e-4
        assert abs(np.mean(codes == 0) - 0.3108) < 0.01


def test_ternarize_exact_tie(env):
    codes, s = run(env, tie_matrix())
    assert s.view(np.uint32) == 0x3FEFFFFF and codes[7, 1000] == 0


def test_ternarize_zero_and_tiny(env):
    codes, s = run(env, np.zeros((8, 64), np.uint16))
    assert s == np.float32(1e-5) and not codes.any()
    tiny = np.full((8, 64), 0x3580, np.uint16)       # 2^-20: mean below the floor
    tiny[::2] |= 0x8000
    codes, s = run(env, tiny)
    assert s == np.float32(1e-5)


def test_ternarize_random_bit_patterns(env):
    # every finite bf16 pattern class: subnormals, normals over the whole
    # exponent range, both zeros; means far above and below 1
    rng = np.random.default_rng(77)
    bits = rng.integers(0, 1 << 16, size=(64, 1024), dtype=np.uint32).astype(np.uint16)
    bits[(bits & 0x7F80) == 0x7F80] &= 0xBFFF            # no Inf/NaN
    run(env, bits)
    small = (bits & 0x83FF) | 0x0000                       # exponents 0..7
    run(env, small.astype(np.uint16))


def test_ternarize_empty(env):
    torch, tq, _ = env
    w = torch.empty(0, 64, dtype=torch.bfloat16, device="cuda")
    packed, s = tq.tq_ternarize(w)
    torch.cuda.synchronize()
    assert packed.shape == (0, 64) and s.cpu().numpy()[0] == np.float32(1e-5)
