"""Graph capture of the library calls that use scratch or several launches:
tq_ternarize (a fill kernel clears its workspace, no memset node),
tq_attn_decode (chunk pass + combine through a workspace) and the grouped
quantize+GEMV.  Each graph is replayed several times with other eager work
and synchronizations in between, and every replay must equal the eager
result bit for bit.
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


def capture(torch, fn):
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()                                   # warm-up outside the graph
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def test_ternarize_graph(env):
    torch, tq = env
    print("graph: ternarize", flush=True)
    bits = workloads.weights_bf16(256, 1024, seed=71)
    w = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).cuda()
    ref_p, ref_s = tq.tq_ternarize(w)
    torch.cuda.synchronize()
    ref_p, ref_s = ref_p.clone(), ref_s.clone()
    packed = torch.empty_like(ref_p)
    scale = torch.empty_like(ref_s)
    ws = torch.empty(tq.TQ_TERNARIZE_WORKSPACE_BYTES, dtype=torch.uint8, device="cuda")
    g = capture(torch, lambda: tq.tq_ternarize(w, packed, scale, ws))
    for rep in range(4):
        packed.fill_(0)
        scale.fill_(0)
        ws.fill_(0xFF)                         # stale workspace contents
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(packed, ref_p), rep
        assert torch.equal(scale.view(torch.int32), ref_s.view(torch.int32)), rep


def test_attn_graph(env):
    torch, tq = env
    print("graph: attention", flush=True)
    torch.manual_seed(72)
    q = torch.randn(20, 128, device="cuda")
    k = torch.randn(3000, 5, 128, device="cuda").to(torch.bfloat16)
    v = torch.randn(3000, 5, 128, device="cuda").to(torch.bfloat16)
    ref = tq.tq_attn_decode(q, k, v)
    torch.cuda.synchronize()
    ref = ref.clone()
    out = torch.empty_like(ref)
    ws = tq.attn_workspace(20, 128, 3000, "cuda")
    g = capture(torch, lambda: tq.tq_attn_decode(q, k, v, out=out, workspace=ws))
    for rep in range(4):
        out.fill_(7.0)
        ws.fill_(0xFF)  # any contents
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int32), ref.view(torch.int32)), rep


def test_group_graph(env):
    torch, tq = env
    print("graph: grouped quant_gemv", flush=True)
    packs = []
    for i, (N, K) in enumerate([(2560, 2560), (640, 2560), (640, 2560)]):
        codes = workloads.ternary_codes(N, K, seed=73 + i)
        packs.append(tq.tq_pack(torch.from_numpy(codes).cuda()))
    xb = workloads.activations_bf16(1, 2560, seed=76, outliers=True)
    x = torch.from_numpy(xb.view(np.int16)).view(torch.bfloat16).cuda()[0]
    scales = [0.02, 0.021, 0.022]
    ref = [t.clone() for t in tq.tq_quant_gemv_group(x, packs, scales)]
    torch.cuda.synchronize()
    ys = [torch.empty_like(t) for t in ref]
    xq = torch.empty(2560, dtype=torch.int8, device="cuda")
    xs = torch.empty(1, dtype=torch.float32, device="cuda")
    g = capture(torch, lambda: tq.tq_quant_gemv_group(x, packs, scales, ys, xq=xq, x_scale=xs))
    for rep in range(4):
        for t in ys:
            t.fill_(3.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip(ys, ref):
            assert torch.equal(a.view(torch.int32), b.view(torch.int32)), rep


def test_rmsnorm_gemv3_dot4_graph(env):
    # one graph with the RMSNorm-fused GEMV, the five-per-byte GEMV and the
    # vector-ALU small batch; every replay must equal the eager results
    torch, tq = env
    print("graph: rmsnorm_quant_gemv, gemv3, gemm_small M=2", flush=True)
    N, K = 2560, 6912
    codes = torch.from_numpy(workloads.ternary_codes(N, K, seed=81)).cuda()
    p2, p3 = tq.tq_pack(codes), tq.tq_pack3(codes)
    xb = workloads.activations_bf16(3, K, seed=82, outliers=True)
    x = torch.from_numpy(xb.view(np.int16)).view(torch.bfloat16).cuda()
    gam = (1.0 + 0.2 * torch.randn(K, device="cuda")).to(torch.bfloat16)
    xq, xs = tq.tq_act_quant(x)
    torch.cuda.synchronize()
    r1 = tq.tq_rmsnorm_quant_gemv(x[0], gam, p2, 0.02).clone()
    r2 = tq.tq_gemv3(p3, 0.02, xq[0], xs[0:1], N).clone()
    q2, s2 = xq[:2].contiguous(), xs[:2].contiguous()
    r3 = tq.tq_gemm_small(p2, 0.02, q2, s2).clone()
    torch.cuda.synchronize()
    y1, y2, y3 = torch.empty_like(r1), torch.empty_like(r2), torch.empty_like(r3)
    q1 = torch.empty(K, dtype=torch.int8, device="cuda")
    s1 = torch.empty(1, dtype=torch.float32, device="cuda")
    xs0 = xs[0:1].clone()

    def work():
        tq.tq_rmsnorm_quant_gemv(x[0], gam, p2, 0.02, y=y1, xq=q1, x_scale=s1)
        tq.tq_gemv3(p3, 0.02, xq[0], xs0, N, y2)
        tq.tq_gemm_small(p2, 0.02, q2, s2, y3)
    g = capture(torch, work)
    for rep in range(4):
        for t in (y1, y2, y3):
            t.fill_(5.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for a, b in ((y1, r1), (y2, r2), (y3, r3)):
            assert torch.equal(a.view(torch.int32), b.view(torch.int32)), rep


def test_gemm_quad_graph(env):
    # the matrix-core small batch in one graph: M = 16 and 64, two shapes, the
    # gated form at M = 32 (dynamic LDS above 64 KB, one and two blocks of
    # partial tiles per wave); every replay must equal the eager results
    torch, tq = env
    print("graph: gemm_small M=16, 64; gate_up M=32", flush=True)
    cases = [(16, 6912, 2560), (64, 2560, 6912)]
    ps, qs, ss, refs = [], [], [], []
    for i, (M, N, K) in enumerate(cases):
        ps.append(tq.tq_pack(torch.from_numpy(workloads.ternary_codes(N, K, seed=91 + i)).cuda()))
        xb = workloads.activations_bf16(M, K, seed=93 + i, outliers=True)
        q, s = tq.tq_act_quant(torch.from_numpy(xb.view(np.int16)).view(torch.bfloat16).cuda())
        qs.append(q)
        ss.append(s)
    pg = tq.tq_pack(torch.from_numpy(workloads.ternary_codes(6912, 2560, seed=95)).cuda())
    pu = tq.tq_pack(torch.from_numpy(workloads.ternary_codes(6912, 2560, seed=96)).cuda())
    xb = workloads.activations_bf16(32, 2560, seed=97, outliers=True)
    qg, sg = tq.tq_act_quant(torch.from_numpy(xb.view(np.int16)).view(torch.bfloat16).cuda())
    torch.cuda.synchronize()
    for p, q, s in zip(ps, qs, ss):
        refs.append(tq.tq_gemm_small(p, 0.02, q, s).clone())
    refs.append(tq.tq_gate_up_relu2(pg, 0.024, pu, 0.025, qg, sg).clone())
    torch.cuda.synchronize()
    ys = [torch.empty_like(r) for r in refs]

    def work():
        for p, q, s, y in zip(ps, qs, ss, ys):
            tq.tq_gemm_small(p, 0.02, q, s, y)
        tq.tq_gate_up_relu2(pg, 0.024, pu, 0.025, qg, sg, ys[-1])
    g = capture(torch, work)
    for rep in range(4):
        for t in ys:
            t.fill_(5.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip(ys, refs):
            assert torch.equal(a.view(torch.int32), b.view(torch.int32)), rep
