"""tq_attn_decode_noalloc (the allocation-free form of tq_attn_decode, for
callers that cannot allocate device memory) against tq_attn_decode.

Both run the same kernels, so the outputs must be bit-identical.  Two calls
in a row share the library's fixed per-GPU scratch: the first fills all of
it (64 query heads x 64 chunks), the second and third are smaller and must
not see its leftovers.  Sizes past the scratch are rejected before launch.
"""
import sys

import numpy as np
import pytest

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def env():
    import torch
    import bit_gemv_tq_amd as tq
    return torch, tq


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def inputs(torch, L, H, Hkv, D, seed):
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    q = torch.randn(H, D, generator=g, device="cuda", dtype=torch.float32)
    k = torch.randn(L, Hkv, D, generator=g, device="cuda").to(torch.bfloat16)
    v = torch.randn(L, Hkv, D, generator=g, device="cuda").to(torch.bfloat16)
    return q, k, v


# (L, H, Hkv, D): the largest scratch use (64 heads x 64 chunks at D = 128),
# then the 2B-4T heads at a short context, then D = 64 over one chunk.
CALLS = [(32768, 64, 8, 128), (2048, 20, 5, 128), (300, 8, 8, 64), (70000, 16, 2, 64)]


def test_noalloc_matches_workspace_form(env):
    torch, tq = env
    for i, (L, H, Hkv, D) in enumerate(CALLS):
        say(f"attn noalloc call {i}: L={L} H={H} Hkv={Hkv} D={D}")
        q, k, v = inputs(torch, L, H, Hkv, D, seed=100 + i)
        out = torch.full((H, D), float("nan"), device="cuda")
        tq.tq_attn_decode_noalloc(q, k, v, out=out)
        ref = tq.tq_attn_decode(q, k, v)
        torch.cuda.synchronize()
        assert torch.isfinite(out).all()
        assert torch.equal(out.view(torch.int32), ref.view(torch.int32)), f"call {i}"


def test_noalloc_rejects_before_launch(env):
    torch, tq = env
    q, k, v = inputs(torch, 64, 72, 9, 128, seed=7)   # H = 72 > 64
    out = torch.zeros(72, 128, device="cuda")
    with pytest.raises(tq.TQError) as e:
        tq.tq_attn_decode_noalloc(q, k, v, out=out)
    assert e.value.status == 2  # TQ_ERR_SHAPE
    torch.cuda.synchronize()
    assert not out.any()
