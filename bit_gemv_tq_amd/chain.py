"""Decode-step chain: a stack of BitNet-b1.58-shaped layers at M = 1.

Each layer is ten library calls on one stream (no host synchronization):
act_quant -> gemv q, k, v -> act_quant(q) -> gemv o -> act_quant(o) ->
gate_up_relu2 -> act_quant(f) -> gemv down.  Buffers are allocated once, so
a whole step can be captured in a HIP graph and replayed.

The page "Feature request: BitNet 1.58-bit ternary inference on ROCm
(gfx1151)", section "Architecture", gives the layer only in outline
(squared-ReLU MLP; sub-layer norms before o_proj and down_proj); attention,
the norms and the residual are not part of this path.  Reading used here:
q's output stands in for the attention output fed to o; k and v are computed
(they would go to the KV cache) but feed nothing; every projection is
rescaled with the unit activation scale 1/127, i.e. its input is taken as
absmax-normalized, standing in for the norms (the plain per-token scales
would drive the activations to zero within a few layers, since relu^2 is
cubic in its input scale).  Compute happens only in the library's kernels.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from . import (tq_act_quant, tq_gate_up_relu2, tq_gemv, tq_quant_gate_up_relu2,
               tq_quant_gemv, tq_quant_gemv_group)

PROJ = ("q", "k", "v", "o", "gate", "up", "down")


@dataclass
class Layer:
    """Packed weights ([N/4, K] uint8 device tensors) and fp32 scales."""
    packed: dict
    scale: dict

    def n(self, name):
        return self.packed[name].shape[0] * 4

    def k(self, name):
        return self.packed[name].shape[1]


class DecodeChain:
    """Preallocated buffers and the launch sequence of one decode step.

    fused=False: ten launches per layer (separate act-quant launches);
    fused=True: four, each launch quantizing its own input in the GEMV
    prologue (q, k and v in one grouped launch, tq_quant_gemv_group; then
    tq_quant_gemv for o and down, tq_quant_gate_up_relu2).  Both give
    bit-identical stages."""

    def __init__(self, layers, device, fused=False):
        self.fused = fused
        import torch
        self.layers = layers
        self.device = device
        L0 = layers[0]
        H, Q, KV, I = L0.k("q"), L0.n("q"), L0.n("k"), L0.n("gate")
        f32, i8 = torch.float32, torch.int8
        e = lambda *s, dt=f32: torch.empty(*s, dtype=dt, device=device)
        self.unit = torch.tensor([np.float32(1.0) / np.float32(127.0)],
                                 dtype=f32, device=device)
        self.q8_in, self.s_in = e(H, dt=i8), e(1)
        self.q, self.k, self.v = e(Q), e(KV), e(KV)
        self.q8_o, self.s_o = e(Q, dt=i8), e(1)
        self.o = e(H)
        self.q8_f, self.s_f = e(H, dt=i8), e(1)
        self.f = e(I)
        self.q8_d, self.s_d = e(I, dt=i8), e(1)
        self.h = [e(H), e(H)]   # ping-pong layer outputs

    def layer(self, L: Layer, h_in, h_out, record=None, stream=None):
        if self.fused:
            self.layer_fused(L, h_in, h_out, record, stream)
            return
        u = self.unit
        tq_act_quant(h_in, self.q8_in, self.s_in, stream=stream)
        tq_gemv(L.packed["q"], L.scale["q"], self.q8_in, u, self.q, stream=stream)
        tq_gemv(L.packed["k"], L.scale["k"], self.q8_in, u, self.k, stream=stream)
        tq_gemv(L.packed["v"], L.scale["v"], self.q8_in, u, self.v, stream=stream)
        tq_act_quant(self.q, self.q8_o, self.s_o, stream=stream)
        tq_gemv(L.packed["o"], L.scale["o"], self.q8_o, u, self.o, stream=stream)
        tq_act_quant(self.o, self.q8_f, self.s_f, stream=stream)
        tq_gate_up_relu2(L.packed["gate"], L.scale["gate"], L.packed["up"],
                         L.scale["up"], self.q8_f, u, self.f, stream=stream)
        tq_act_quant(self.f, self.q8_d, self.s_d, stream=stream)
        tq_gemv(L.packed["down"], L.scale["down"], self.q8_d, u, h_out,
                stream=stream)
        if record is not None:
            record.append({name: getattr(self, name).clone() for name in
                           ("q8_in", "s_in", "q", "k", "v", "q8_o", "o", "q8_f",
                            "f", "q8_d")} | {"h": h_out.clone()})

    def layer_fused(self, L: Layer, h_in, h_out, record=None, stream=None):
        u, st = self.unit, stream
        tq_quant_gemv_group(h_in, [L.packed[n] for n in ("q", "k", "v")],
                            [L.scale[n] for n in ("q", "k", "v")],
                            [self.q, self.k, self.v], xq=self.q8_in,
                            x_scale=self.s_in, y_scale=u, stream=st)
        tq_quant_gemv(self.q, L.packed["o"], L.scale["o"], self.o,
                      xq=self.q8_o, x_scale=self.s_o, y_scale=u, stream=st)
        tq_quant_gate_up_relu2(self.o, L.packed["gate"], L.scale["gate"],
                               L.packed["up"], L.scale["up"], self.f,
                               xq=self.q8_f, x_scale=self.s_f, y_scale=u,
                               stream=st)
        tq_quant_gemv(self.f, L.packed["down"], L.scale["down"], h_out,
                      xq=self.q8_d, x_scale=self.s_d, y_scale=u, stream=st)
        if record is not None:
            record.append({name: getattr(self, name).clone() for name in
                           ("q8_in", "s_in", "q", "k", "v", "q8_o", "o", "q8_f",
                            "f", "q8_d")} | {"h": h_out.clone()})

    def step(self, h0, record=None, stream=None):
        """Run every layer from h0 (bf16 or fp32 [H]); returns the output
        buffer holding the last layer's h (overwritten by the next step)."""
        h_in = h0
        for i, L in enumerate(self.layers):
            h_out = self.h[i % 2]
            self.layer(L, h_in, h_out, record, stream)
            h_in = h_out
        return h_in
