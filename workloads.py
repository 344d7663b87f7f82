"""Seeded synthetic inputs and workload shapes for the ternary GEMV path.

This module is shared by the tests, the smoke check and the benchmark.  It
holds no arithmetic of the method itself (no packing, quantization, product
or rescale): only shapes, seeds and random draws.

Shapes follow the 2B-4T weight map on the page "Feature request: BitNet
1.58-bit ternary inference on ROCm (gfx1151)", section "Weight mapping
(bitnet-b1.58-2B-4T)": hidden 2560, intermediate 6912, 20 heads, 5 KV heads,
head_dim 128.  Larger 8B- and 70B-class layer shapes and all value
distributions are synthetic stand-ins (no weights or datasets are used).

Distributions:
  * weights: iid ternary, P(0) = 0.35, P(-1) = P(+1) = 0.325, drawn as one
    uniform per weight against the thresholds 0.325 and 0.675;
  * activations: fp32 standard normal, rounded to bf16 (round-half-even);
  * outliers: exactly max(1, round(0.001*K)) positions per row, drawn without
    replacement, scaled by 20 before the bf16 rounding.
Seeds: seed = 1000 * config + tensor index (+ 100 * layer for the chain).
"""
from __future__ import annotations

import numpy as np

HIDDEN = 2560
INTERMEDIATE = 6912
N_HEADS = 20
N_KV_HEADS = 5
HEAD_DIM = 128
KV_DIM = N_KV_HEADS * HEAD_DIM  # 640

P_ZERO = 0.35
P_NEG = (1.0 - P_ZERO) / 2.0

# The seven projections of one 2B-4T layer: name -> (N outputs, K inputs).
LAYER_2B4T = {
    "q": (HIDDEN, HIDDEN),
    "k": (KV_DIM, HIDDEN),
    "v": (KV_DIM, HIDDEN),
    "o": (HIDDEN, HIDDEN),
    "gate": (INTERMEDIATE, HIDDEN),
    "up": (INTERMEDIATE, HIDDEN),
    "down": (HIDDEN, INTERMEDIATE),
}
TENSOR_INDEX = {name: t for t, name in enumerate(LAYER_2B4T)}

# A 70B-class layer for the decode chain at the large shapes: hidden 8192,
# intermediate 28672 (the 70B-class shapes above), q/o [8192, 8192] and
# grouped-query k/v of 8 heads x 128 = 1024 rows.  Same projection names,
# so TENSOR_INDEX applies.
LAYER_70B = {
    "q": (8192, 8192),
    "k": (1024, 8192),
    "v": (1024, 8192),
    "o": (8192, 8192),
    "gate": (28672, 8192),
    "up": (28672, 8192),
    "down": (8192, 28672),
}
CHAIN_70B_CONFIG = 7  # seed_for config id of its weights and input

# 8B- and 70B-class M=1 layers, both orientations: (N, K).
LARGE_SHAPES = {
    "8b_up": (14336, 4096),
    "8b_down": (4096, 14336),
    "70b_up": (28672, 8192),
    "70b_down": (8192, 28672),
}

# Small-batch GEMM cases: M in {4, 16, 64} x these (N, K).
GEMM_SMALL_M = (4, 16, 64)
GEMM_SMALL_SHAPES = ((INTERMEDIATE, HIDDEN), (HIDDEN, INTERMEDIATE))

CHAIN_LAYERS = 30


def tensor_scale(t: int) -> np.float32:
    """Per-tensor weight scale: 0.020 + 0.001 * tensor index (0.02 for t=0)."""
    return np.float32(0.020 + 0.001 * t)


def seed_for(config: int, tensor: int = 0, layer: int = 0) -> int:
    return 1000 * config + 100 * layer + tensor


def ternary_codes(N: int, K: int, seed: int, p_zero: float = P_ZERO) -> np.ndarray:
    """iid ternary weights [N, K] int8 with P(0) = p_zero."""
    rng = np.random.default_rng(seed)
    out = np.empty((N, K), np.int8)
    p_neg = (1.0 - p_zero) / 2.0
    lo, hi = np.float32(p_neg), np.float32(p_neg + p_zero)
    rows = max(1, (1 << 24) // max(K, 1))
    for r0 in range(0, N, rows):
        u = rng.random((min(rows, N - r0), K), dtype=np.float32)
        blk = out[r0:r0 + u.shape[0]]
        blk[...] = (u >= lo).astype(np.int8)
        blk += (u >= hi).astype(np.int8)
        blk -= 1
    return out


def ternary_codes_torch(N: int, K: int, seed: int, device, p_zero: float = P_ZERO):
    """Same distribution as ternary_codes, drawn with torch's generator on
    ``device`` (used where numpy generation on the host would be too slow)."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    u = torch.rand((N, K), generator=g, device=device, dtype=torch.float32)
    p_neg = (1.0 - p_zero) / 2.0
    w = (u >= p_neg).to(torch.int8)
    w += (u >= p_neg + p_zero).to(torch.int8)
    w -= 1
    del u
    return w


def normal_f32(M: int, K: int, seed: int, outliers: bool = False) -> np.ndarray:
    """fp32 N(0,1) [M, K]; optionally max(1, round(0.001 K)) entries per row
    scaled by 20 (positions without replacement)."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((M, K), dtype=np.float32)
    if outliers and K > 0:
        n_out = max(1, int(round(0.001 * K)))
        for m in range(M):
            idx = rng.choice(K, size=n_out, replace=False)
            x[m, idx] *= np.float32(20.0)
    return x


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 (round-half-even) bit patterns as uint16, via torch CPU."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


def activations_bf16(M: int, K: int, seed: int, outliers: bool = False) -> np.ndarray:
    """Synthetic bf16 activations [M, K] as uint16 bit patterns."""
    return to_bf16_bits(normal_f32(M, K, seed, outliers))


def weights_bf16(N: int, K: int, seed: int, sigma: float = 0.02) -> np.ndarray:
    """Synthetic pre-dequantized weights [N, K]: fp32 N(0, sigma^2) rounded
    to bf16 (uint16 bit patterns), the input of the absmean ternarizer."""
    rng = np.random.default_rng(seed)
    w = rng.standard_normal((N, K), dtype=np.float32) * np.float32(sigma)
    return to_bf16_bits(w)
