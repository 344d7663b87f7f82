"""GPU parity of the decode-step chain: 30 layers of 2B-4T-shaped ternary
projections at M = 1 with per-token re-quantization between projections,
against the oracle's chain on the same seeded weights and input (bf16 N(0,1)
with 0.1% of entries scaled by 20).  Every stage of every layer is compared:
int8 activations and int32-derived fp32 outputs bit for bit.
"""
import numpy as np
import pytest

import workloads

pytestmark = pytest.mark.gpu


def build_layers(torch, tq, oracle, n_layers, cfg=2, shapes=None):
    from bit_gemv_tq_amd.chain import Layer
    shapes = shapes or workloads.LAYER_2B4T
    dev_layers, ref_layers = [], []
    for l in range(n_layers):
        packed, scale, ref = {}, {}, {}
        for name, (N, K) in shapes.items():
            t = workloads.TENSOR_INDEX[name]
            codes = workloads.ternary_codes(N, K, seed=workloads.seed_for(cfg, t, l))
            w = torch.from_numpy(codes).cuda()
            packed[name] = tq.tq_pack(w)
            del w
            scale[name] = workloads.tensor_scale(t)
            ref[name] = (oracle.pack(codes), scale[name], N)
        dev_layers.append(Layer(packed, scale))
        ref_layers.append(ref)
    return dev_layers, ref_layers


@pytest.mark.parametrize("n_layers,graph,fused", [(3, False, False), (30, False, False),
                                                   (30, True, False), (30, False, True),
                                                   (30, True, True)])
def test_chain(n_layers, graph, fused):
    import torch
    import bit_gemv_tq_amd as tq
    import oracle
    from bit_gemv_tq_amd.chain import DecodeChain

    print(f"chain layers={n_layers} graph={graph} fused={fused}", flush=True)
    dev_layers, ref_layers = build_layers(torch, tq, oracle, n_layers)
    h0 = workloads.activations_bf16(1, workloads.HIDDEN, seed=workloads.seed_for(2, 9),
                                    outliers=True)
    h0_dev = torch.from_numpy(h0.view(np.int16)).view(torch.bfloat16).cuda()[0]
    chain = DecodeChain(dev_layers, "cuda", fused=fused)
    h_ref, st_ref = oracle.decode_chain(ref_layers, h0, keep_stages=True)

    if not graph:
        rec = []
        out = chain.step(h0_dev, record=rec)
        torch.cuda.synchronize()
        for l, (g, r) in enumerate(zip(rec, st_ref)):
            for key in ("q8_in", "q8_o", "q8_f", "q8_d"):
                np.testing.assert_array_equal(g[key].cpu().numpy(), r[key][0],
                                              err_msg=f"layer {l} {key}")
            for key in ("q", "k", "v", "o", "f", "h"):
                np.testing.assert_array_equal(
                    g[key].cpu().numpy().view(np.uint32), r[key][0].view(np.uint32),
                    err_msg=f"layer {l} {key}")
        np.testing.assert_array_equal(out.cpu().numpy().view(np.uint32),
                                      h_ref[0].view(np.uint32))
        assert np.abs(h_ref).max() > 1e-3      # the chain did not collapse
        return

    # Graph capture of one whole step, replayed several times with eager work
    # and synchronizations in between; every replay must equal the eager run.
    eager = chain.step(h0_dev).clone()
    torch.cuda.synchronize()
    np.testing.assert_array_equal(eager.cpu().numpy().view(np.uint32),
                                  h_ref[0].view(np.uint32))
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        chain.step(h0_dev)                        # warm-up on the side stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        out = chain.step(h0_dev)
    for rep in range(4):
        chain.h[0].fill_(3.0)
        chain.h[1].fill_(-1.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        np.testing.assert_array_equal(out.cpu().numpy().view(np.uint32),
                                      h_ref[0].view(np.uint32), err_msg=f"replay {rep}")


def test_chain_70b_layer():
    """One 70B-class layer (grouped q/k/v [8192, 1024, 1024] x 8192, o
    [8192, 8192], gate/up [28672, 8192], down [8192, 28672]) through the
    fused chain, every stage bit for bit against the oracle."""
    import torch
    import bit_gemv_tq_amd as tq
    import oracle
    from bit_gemv_tq_amd.chain import DecodeChain

    cfg = workloads.CHAIN_70B_CONFIG
    print("chain 70B-class layer, fused", flush=True)
    dev_layers, ref_layers = build_layers(torch, tq, oracle, 1, cfg=cfg,
                                          shapes=workloads.LAYER_70B)
    H = workloads.LAYER_70B["q"][1]
    h0 = workloads.activations_bf16(1, H, seed=workloads.seed_for(cfg, 9), outliers=True)
    h0_dev = torch.from_numpy(h0.view(np.int16)).view(torch.bfloat16).cuda()[0]
    chain = DecodeChain(dev_layers, "cuda", fused=True)
    h_ref, st_ref = oracle.decode_chain(ref_layers, h0, keep_stages=True)
    rec = []
    out = chain.step(h0_dev, record=rec)
    torch.cuda.synchronize()
    g, r = rec[0], st_ref[0]
    for key in ("q8_in", "q8_o", "q8_f", "q8_d"):
        np.testing.assert_array_equal(g[key].cpu().numpy(), r[key][0], err_msg=key)
    for key in ("q", "k", "v", "o", "f", "h"):
        np.testing.assert_array_equal(g[key].cpu().numpy().view(np.uint32),
                                      r[key][0].view(np.uint32), err_msg=key)
    np.testing.assert_array_equal(out.cpu().numpy().view(np.uint32),
                                  h_ref[0].view(np.uint32))
    assert np.abs(h_ref).max() > 1e-3
