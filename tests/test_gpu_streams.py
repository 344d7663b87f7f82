"""Library calls on two streams at once.

Every call takes its stream and touches only the buffers it is given (and,
for tq_attn_decode, the workspace it is given), so calls on different
streams may overlap.  Two streams run different calls back to back many
times over, with no ordering between them; every result must equal the one
the same call gave alone, bit for bit.  (The fixed per-GPU scratch of
tq_attn_decode_noalloc is the documented exception and is not used here.)
"""
import numpy as np
import pytest

import workloads

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def env():
    import torch
    import bit_gemv_tq_amd as tq
    return torch, tq


def bits(t):
    """Host copy of a result: fp32 as its bit patterns, integers as they are."""
    a = t.cpu().numpy()
    return a.view(np.uint32) if a.dtype == np.float32 else a


def test_two_streams(env):
    torch, tq = env
    print("two streams", flush=True)
    dev = torch.device("cuda")
    pa = tq.tq_pack(workloads.ternary_codes_torch(8192, 8192, seed=91, device=dev))
    pg = tq.tq_pack(workloads.ternary_codes_torch(6912, 2560, seed=92, device=dev))
    pu = tq.tq_pack(workloads.ternary_codes_torch(6912, 2560, seed=93, device=dev))
    pm = tq.tq_pack(workloads.ternary_codes_torch(2560, 6912, seed=94, device=dev))
    xa = torch.from_numpy(workloads.activations_bf16(1, 8192, seed=95).view(np.int16)) \
        .view(torch.bfloat16).to(dev)[0]
    xb = torch.from_numpy(workloads.activations_bf16(16, 6912, seed=96).view(np.int16)) \
        .view(torch.bfloat16).to(dev)
    xg = torch.from_numpy(workloads.activations_bf16(1, 2560, seed=97).view(np.int16)) \
        .view(torch.bfloat16).to(dev)[0]
    g = torch.Generator(device=dev).manual_seed(98)
    q = torch.randn(20, 128, generator=g, device=dev)
    kc = torch.randn(4096, 5, 128, generator=g, device=dev).to(torch.bfloat16)
    vc = torch.randn(4096, 5, 128, generator=g, device=dev).to(torch.bfloat16)

    def stream_a(o):
        # fused quantize + GEMV, then gate/up + relu^2 on the quantized row
        # of another activation (act-quant + gate call)
        tq.tq_quant_gemv(xa, pa, 0.02, y=o["ya"], acc=o["acc_a"], xq=o["xq_a"],
                         x_scale=o["xs_a"])
        tq.tq_act_quant(xg[None], xq=o["xq_g"], x_scale=o["xs_g"])
        tq.tq_gate_up_relu2(pg, 0.03, pu, 0.04, o["xq_g"], o["xs_g"], h=o["h"])

    def stream_b(o):
        # act-quant of 16 rows + the matrix-core GEMM, then decode attention
        tq.tq_act_quant(xb, xq=o["xq_b"], x_scale=o["xs_b"])
        tq.tq_gemm_small(pm, 0.05, o["xq_b"], o["xs_b"], y=o["yb"])
        tq.tq_attn_decode(q, kc, vc, out=o["att"], workspace=o["ws"])

    def outputs():
        return {
            "ya": torch.empty(8192, device=dev),
            "acc_a": torch.empty(8192, dtype=torch.int32, device=dev),
            "xq_a": torch.empty(8192, dtype=torch.int8, device=dev),
            "xs_a": torch.empty(1, device=dev),
            "xq_g": torch.empty(1, 2560, dtype=torch.int8, device=dev),
            "xs_g": torch.empty(1, device=dev),
            "h": torch.empty(1, 6912, device=dev),
            "xq_b": torch.empty(16, 6912, dtype=torch.int8, device=dev),
            "xs_b": torch.empty(16, device=dev),
            "yb": torch.empty(16, 2560, device=dev),
            "att": torch.empty(20, 128, device=dev),
            "ws": tq.attn_workspace(20, 128, 4096, dev),
        }

    ref = outputs()
    stream_a(ref)
    torch.cuda.synchronize()
    stream_b(ref)
    torch.cuda.synchronize()
    keys = [k for k in ref if k != "ws"]
    want = {k: bits(ref[k]) for k in keys}

    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()
    sa.wait_stream(torch.cuda.current_stream())
    sb.wait_stream(torch.cuda.current_stream())
    oa, ob = outputs(), outputs()
    for rnd in range(3):
        for o in (oa, ob):
            for k in keys:
                o[k].fill_(-1 if o[k].dtype != torch.int8 else 0)
        torch.cuda.synchronize()
        with torch.cuda.stream(sa):
            for _ in range(20):
                stream_a(oa)
        with torch.cuda.stream(sb):
            for _ in range(20):
                stream_b(ob)
        torch.cuda.synchronize()
        for k in ("ya", "acc_a", "xq_a", "xs_a", "xq_g", "xs_g", "h"):
            np.testing.assert_array_equal(bits(oa[k]), want[k], err_msg=f"{k} round {rnd}")
        for k in ("xq_b", "xs_b", "yb", "att"):
            np.testing.assert_array_equal(bits(ob[k]), want[k], err_msg=f"{k} round {rnd}")
