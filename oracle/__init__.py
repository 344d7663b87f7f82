"""CPU oracle for the BitNet b1.58 ternary GEMV hot path.

TEST INFRASTRUCTURE ONLY.  Only the test suite, ``__graft_entry__.smoke()``
and the CPU-baseline leg of ``bench.py`` may import this package.  The product
path (``bit_gemv_tq_amd`` and its HIP library) never imports it, and the two
share no code: the arithmetic here lives in ``tq_oracle.c`` (plain C, gcc),
wrapped with ctypes over numpy arrays.

Pages cited by title:
  [ISSUE]  "Feature request: BitNet 1.58-bit ternary inference on ROCm
           (gfx1151)": sections "Architecture" (relu^2 MLP, sub-layer norms
           before o_proj and down_proj, uint8 packing with four values per
           byte) and "Weight mapping (bitnet-b1.58-2B-4T)" (the seven
           projection shapes and their packed [N/4, K] uint8 forms).

Function-by-function definitions are in ``tq_oracle.h``.  Every function
here is pinned by a ``-m "not gpu"`` test except where its docstring says
"parity unpinned".
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "tq_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libtq_oracle.so")

GCC_FLAGS = ["-O2", "-fno-fast-math", "-ffp-contract=off", "-std=c11",
             "-Wall", "-Wextra", "-shared", "-fPIC"]

_ERRORS = {1: "bad argument", 2: "bad shape (N % 4 != 0)",
           3: "bad ternary value or reserved code 3",
           4: "accumulator out of int32 range"}


class OracleError(RuntimeError):
    pass


def build(force: bool = False) -> str:
    """Compile tq_oracle.c with gcc into libtq_oracle.so (in-tree)."""
    if force or not os.path.exists(_LIB_PATH) or \
            os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", *GCC_FLAGS, _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        build()
        L = ctypes.CDLL(_LIB_PATH)
        i64, p = ctypes.c_int64, ctypes.c_void_p
        L.tqo_bf16_to_f32.argtypes = [ctypes.c_uint16]
        L.tqo_bf16_to_f32.restype = ctypes.c_float
        sig = {
            "tqo_pack": [p, i64, i64, p],
            "tqo_unpack": [p, i64, i64, p],
            "tqo_pack3": [p, i64, i64, p],
            "tqo_unpack3": [p, i64, i64, p],
            "tqo_act_quant_f32": [p, i64, i64, p, p],
            "tqo_act_quant_bf16": [p, i64, i64, p, p],
            "tqo_rmsnorm_act_quant_f32": [p, p, ctypes.c_float, i64, i64, p, p],
            "tqo_rmsnorm_act_quant_bf16": [p, p, ctypes.c_float, i64, i64, p, p],
            "tqo_ternary_matmul": [p, p, i64, i64, i64, p],
            "tqo_ternary_matmul_rows": [p, p, i64, i64, i64, p, i64, p],
            "tqo_rescale_f32": [p, ctypes.c_float, p, i64, i64, p],
            "tqo_rescale_f64": [p, ctypes.c_float, p, i64, i64, p],
            "tqo_relu2_f32": [p, p, i64, p],
            "tqo_relu2_f64": [p, p, i64, p],
        }
        for name, args in sig.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = ctypes.c_int
        _lib = L
    return _lib


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p) if a.size else None


def _check(rc: int, what: str):
    if rc:
        raise OracleError(f"{what}: {_ERRORS.get(rc, rc)}")


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


# --------------------------------------------------------------------------
# primitives
# --------------------------------------------------------------------------
def bf16_to_f32(bits) -> np.ndarray:
    """bf16 bit patterns (uint16) -> fp32, one element at a time in C."""
    bits = _c(bits, np.uint16)
    f = lib().tqo_bf16_to_f32
    out = np.empty(bits.shape, np.float32)
    flat = out.reshape(-1)
    for i, b in enumerate(bits.reshape(-1)):
        flat[i] = f(int(b))
    return out


def pack(w) -> np.ndarray:
    """int8 ternary weights [N, K] -> packed uint8 [N/4, K] ([ISSUE] uint8,
    four values per byte; plane j of byte [i, k] holds row j*N/4 + i)."""
    w = _c(w, np.int8)
    N, K = w.shape
    out = np.zeros((N // 4, K), np.uint8)
    _check(lib().tqo_pack(_ptr(w), N, K, _ptr(out)), "pack")
    return out


def unpack(packed, N: int) -> np.ndarray:
    packed = _c(packed, np.uint8)
    K = packed.shape[1]
    out = np.zeros((N, K), np.int8)
    _check(lib().tqo_unpack(_ptr(packed), N, K, _ptr(out)), "unpack")
    return out


def pack3(w) -> np.ndarray:
    """int8 weights [N, K] in {-1,0,1} -> uint8 [ceil(N/5), K], five weights
    per byte (base 3, stored as ceil(256 v / 243))."""
    w = _c(w, np.int8)
    N, K = w.shape
    out = np.zeros(((N + 4) // 5, K), np.uint8)
    _check(lib().tqo_pack3(_ptr(w), N, K, _ptr(out)), "pack3")
    return out


def unpack3(packed, N: int) -> np.ndarray:
    packed = _c(packed, np.uint8)
    K = packed.shape[1]
    if packed.shape[0] != (N + 4) // 5:
        raise ValueError(f"packed has {packed.shape[0]} rows, need ceil({N}/5)")
    out = np.zeros((N, K), np.int8)
    _check(lib().tqo_unpack3(_ptr(packed), N, K, _ptr(out)), "unpack3")
    return out


def act_quant(x, dtype: str = "bf16"):
    """Per-row absmax int8 quantization.  ``x`` is [M, K]: uint16 bf16 bit
    patterns when dtype == 'bf16', fp32 values when dtype == 'f32'.
    Returns (q int8 [M, K], s_x fp32 [M])."""
    if dtype == "bf16":
        x = _c(x, np.uint16)
        fn = lib().tqo_act_quant_bf16
    elif dtype == "f32":
        x = _c(x, np.float32)
        fn = lib().tqo_act_quant_f32
    else:
        raise ValueError(dtype)
    if x.ndim == 1:
        x = x.reshape(1, -1)
    M, K = x.shape
    q = np.zeros((M, K), np.int8)
    s = np.zeros((M,), np.float32)
    _check(fn(_ptr(x), M, K, _ptr(q), _ptr(s) if M else None), "act_quant")
    return q, s


def rmsnorm_act_quant(x, gamma, eps: float, dtype: str = "bf16"):
    """Sub-layer RMSNorm folded into per-row absmax quantization ([ISSUE]
    "Architecture": norms before o_proj and down_proj).  ``x`` [M, K] and
    ``gamma`` [K] are uint16 bf16 bit patterns (dtype 'bf16') or fp32.
    Returns (q int8 [M, K], s_x fp32 [M]): q are the codes of x*gamma and
    s_x = (a'/127) / sqrt(mean(x^2) + eps), so q * s_x approximates
    RMSNorm(x) * gamma."""
    dt = {"bf16": np.uint16, "f32": np.float32}[dtype]
    x = _c(x, dt)
    gamma = _c(gamma, dt).reshape(-1)
    if x.ndim == 1:
        x = x.reshape(1, -1)
    M, K = x.shape
    if gamma.size != K:
        raise ValueError("gamma must have K entries")
    q = np.zeros((M, K), np.int8)
    s = np.zeros((M,), np.float32)
    fn = (lib().tqo_rmsnorm_act_quant_bf16 if dtype == "bf16"
          else lib().tqo_rmsnorm_act_quant_f32)
    _check(fn(_ptr(x), _ptr(gamma), float(np.float32(eps)), M, K, _ptr(q),
              _ptr(s) if M else None), "rmsnorm_act_quant")
    return q, s


def ternary_matmul(packed, q, N: int) -> np.ndarray:
    """acc[m, n] = sum_k W[n, k] q[m, k] (exact int, asserted to fit int32)."""
    packed = _c(packed, np.uint8)
    q = _c(q, np.int8)
    if q.ndim == 1:
        q = q.reshape(1, -1)
    M, K = q.shape
    if packed.shape != (N // 4, K):
        raise ValueError(f"packed shape {packed.shape} != {(N // 4, K)}")
    acc = np.zeros((M, N), np.int32)
    _check(lib().tqo_ternary_matmul(_ptr(packed), _ptr(q), M, N, K,
                                    _ptr(acc)), "ternary_matmul")
    return acc


def ternary_matmul_rows(packed, q, N: int, rows) -> np.ndarray:
    """Like ternary_matmul, for output rows ``rows`` only: acc [M, len(rows)]."""
    packed = _c(packed, np.uint8)
    q = _c(q, np.int8)
    if q.ndim == 1:
        q = q.reshape(1, -1)
    rows = _c(rows, np.int64)
    M, K = q.shape
    acc = np.zeros((M, rows.size), np.int32)
    _check(lib().tqo_ternary_matmul_rows(_ptr(packed), _ptr(q), M, N, K,
                                         _ptr(rows), rows.size, _ptr(acc)),
           "ternary_matmul_rows")
    return acc


def rescale(acc, s_w: float, s_x, exact: bool = False) -> np.ndarray:
    """y = acc * s_w * s_x[m]: fp32 in the fixed order, or exact (fp64)."""
    acc = _c(acc, np.int32)
    if acc.ndim == 1:
        acc = acc.reshape(1, -1)
    s_x = _c(s_x, np.float32).reshape(-1)
    M, N = acc.shape
    if exact:
        y = np.zeros((M, N), np.float64)
        fn = lib().tqo_rescale_f64
    else:
        y = np.zeros((M, N), np.float32)
        fn = lib().tqo_rescale_f32
    _check(fn(_ptr(acc), float(np.float32(s_w)), _ptr(s_x), M, N, _ptr(y)),
           "rescale")
    return y


def relu2(g, u, exact: bool = False) -> np.ndarray:
    """h = relu(g)^2 * u ([ISSUE] "Architecture": squared-ReLU MLP)."""
    dt = np.float64 if exact else np.float32
    g = _c(g, dt)
    u = _c(u, dt)
    if g.shape != u.shape:
        raise ValueError("shape mismatch")
    h = np.zeros(g.shape, dt)
    fn = lib().tqo_relu2_f64 if exact else lib().tqo_relu2_f32
    _check(fn(_ptr(g), _ptr(u), g.size, _ptr(h)), "relu2")
    return h


# --------------------------------------------------------------------------
# compositions (each a short sequence of the primitives above)
# --------------------------------------------------------------------------
def gemv(packed, s_w: float, q, s_x, N: int, exact: bool = False):
    """One ternary projection: (acc int32 [M, N], y [M, N])."""
    acc = ternary_matmul(packed, q, N)
    return acc, rescale(acc, s_w, s_x, exact=exact)


def gate_up_relu2(packed_g, s_g, packed_u, s_u, q, s_x, N: int,
                  exact: bool = False):
    """Fused gate/up projection with relu^2: (acc_g, acc_u, h)."""
    acc_g, g = gemv(packed_g, s_g, q, s_x, N, exact)
    acc_u, u = gemv(packed_u, s_u, q, s_x, N, exact)
    return acc_g, acc_u, relu2(g, u, exact)


UNIT_SCALE = np.float32(1.0) / np.float32(127.0)


def decode_layer(layer, h_in, h_dtype: str = "f32"):
    """One layer of the decode-step chain, as a dict of every stage.

    ``layer`` maps 'q','k','v','o','gate','up','down' to (packed, s_w, N).
    The pages give the layer only in outline ([ISSUE] "Architecture": squared
    ReLU MLP, sub-layer norms before o_proj and down_proj); attention, norms
    and the residual are not part of this path.  Reading used: every
    projection input is re-quantized per token, q's output stands in for the
    attention output fed to o, and every projection is rescaled with the unit
    activation scale 1/127 (the input taken as absmax-normalized, standing in
    for the sub-layer norms), so that relu^2 does not drive the activations to
    zero within a few layers.  k and v are computed and returned but feed
    nothing (they would go to the KV cache).
    """
    one = np.array([UNIT_SCALE], np.float32)
    st = {}
    st["q8_in"], st["s_in"] = act_quant(h_in, h_dtype)
    for name in ("q", "k", "v"):
        p, s_w, N = layer[name]
        st["acc_" + name], st[name] = gemv(p, s_w, st["q8_in"], one, N)
    st["q8_o"], st["s_o"] = act_quant(st["q"], "f32")
    p, s_w, N = layer["o"]
    st["acc_o"], st["o"] = gemv(p, s_w, st["q8_o"], one, N)
    st["q8_f"], st["s_f"] = act_quant(st["o"], "f32")
    pg, s_g, Ni = layer["gate"]
    pu, s_u, _ = layer["up"]
    st["acc_gate"], st["acc_up"], st["f"] = gate_up_relu2(
        pg, s_g, pu, s_u, st["q8_f"], one, Ni)
    st["q8_d"], st["s_d"] = act_quant(st["f"], "f32")
    p, s_w, N = layer["down"]
    st["acc_down"], st["h"] = gemv(p, s_w, st["q8_d"], one, N)
    return st


def decode_chain(layers, h0_bf16, keep_stages: bool = False):
    """The decode-step chain over ``layers`` starting from bf16 bits h0.
    Returns the final fp32 h [1, H] and, if asked, every layer's stages."""
    stages = []
    h, dt = h0_bf16, "bf16"
    for layer in layers:
        st = decode_layer(layer, h, dt)
        h, dt = st["h"], "f32"
        stages.append(st if keep_stages else {"h": st["h"]})
    return h, stages


# --------------------------------------------------------------------------
# Absmean ternarization of bf16 weights (the step before packing).
#
# Page "1bit.systems" project README, section "read more": the project's
# training runs use absmean quantization-aware training; page "Feature
# request: BitNet 1.58-bit ternary inference on ROCm (gfx1151)", section
# "Architecture": checkpoints come either as packed uint8 or as
# pre-dequantized bf16.  The pages give no formula.  Reading used (the
# BitNet b1.58 absmean rule, written so that every decision is exact):
#   s   = RN32(mean_{n,k} |w[n,k]|)       (exact sum, one rounding)
#   s'  = max(s, 1e-5f)
#   inv = RN32(1 / s')
#   c   = clamp(rne(RN32(w * inv)), -1, 1)
# and s' is the weight scale (real weight = s' * c).
# --------------------------------------------------------------------------
from fractions import Fraction as _Fraction

_F32_MIN_EXP = -126      # smallest normal binary32 exponent
_F32_P = 24              # binary32 significand bits


def rn32_fraction(v) -> np.float32:
    """Round an exact rational to binary32, ties to even (IEEE 754
    roundTiesToEven, gradual underflow); magnitudes above the largest finite
    value are out of scope here (weights are finite bf16)."""
    v = _Fraction(v)
    if v == 0:
        return np.float32(0.0)
    sign = -1 if v < 0 else 1
    a = abs(v)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if _Fraction(2) ** e > a:
        e -= 1
    elif _Fraction(2) ** (e + 1) <= a:
        e += 1
    ulp = _Fraction(2) ** (max(e, _F32_MIN_EXP) - (_F32_P - 1))
    m = a / ulp
    fl = m.numerator // m.denominator
    rem = m - fl
    if rem > _Fraction(1, 2) or (rem == _Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    return np.float32(sign * float(fl * ulp))


def abs_sum_bf16(w_bits) -> _Fraction:
    """Exact sum of |w| over bf16 bit patterns (uint16/int16, any shape).
    |w| = M * 2^(max(e,1) - 134) with e the 8-bit exponent field and M the
    significand (hidden bit included for e >= 1); the sum is taken exactly
    as an integer multiple of 2^-133, grouping equal exponents."""
    b = np.asarray(w_bits).view(np.uint16).ravel().astype(np.int64)
    e = (b >> 7) & 0xFF
    if np.any(e == 0xFF):
        raise OracleError("Inf/NaN weights are outside the contract")
    m = (b & 0x7F) | np.where(e > 0, 0x80, 0)
    total = 0
    for ev in np.unique(e):
        total += int(m[e == ev].sum(dtype=np.int64)) << (max(int(ev), 1) - 1)
    return _Fraction(total, 1 << 133)


def absmean_scale(w_bits) -> np.float32:
    """s' = max(RN32(sum |w| / count), 1e-5f), exact sum, one rounding."""
    n = np.asarray(w_bits).size
    if n == 0:
        return np.float32(1e-5)
    s = rn32_fraction(abs_sum_bf16(w_bits) / n)
    return max(s, np.float32(1e-5))


def ternarize(w_bits):
    """bf16 weights [N, K] -> (codes int8 [N, K] in {-1, 0, 1}, s')."""
    s = absmean_scale(w_bits)
    inv = np.float32(1.0) / s                      # RN32 division
    # bf16 -> fp32 is exact: the bf16 pattern is the top half of the fp32 one
    w = (np.asarray(w_bits).view(np.uint16).astype(np.uint32) << 16).view(np.float32)
    y = (w * inv).astype(np.float32)               # RN32 product
    codes = np.clip(np.rint(y), -1, 1).astype(np.int8)
    return codes, s


# --------------------------------------------------------------------------
# Split-KV (flash-decoding) attention at decode: the reference result.
#
# Page "1bit.systems" project README, section "honest numbers": split-KV
# Flash-Decoding attention at L = 2048; page "Feature request: BitNet 1.58-bit
# ternary inference on ROCm (gfx1151)", section "Weight mapping": 20 query
# heads, 5 KV heads, head_dim 128 (grouped-query attention).  The pages give
# no formula or precision; reading used (standard scaled dot-product
# attention for one query token over L cached tokens, no mask):
#   s[h,t] = scale * sum_d q[h,d] * k[t,g,d],   g = h // (H / Hkv)
#   o[h,:] = sum_t softmax_t(s[h,:]) * v[t,g,:]
# q is fp32 [H, D]; k and v are bf16 [L, Hkv, D] (a token-major KV cache).
# The oracle evaluates this definition in float64 (exact bf16 widening).
# --------------------------------------------------------------------------
def attn_decode(q, k_bits, v_bits, scale) -> np.ndarray:
    """float64 [H, D] attention output of one query token (see above)."""
    q = np.asarray(q, np.float32)
    k_bits = np.asarray(k_bits).view(np.uint16)
    v_bits = np.asarray(v_bits).view(np.uint16)
    H, D = q.shape
    L, Hkv, Dk = k_bits.shape
    if Dk != D or v_bits.shape != k_bits.shape or L < 1 or H % Hkv:
        raise OracleError("bad attention shapes")
    widen = lambda b: (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    k, v = widen(k_bits), widen(v_bits)
    G = H // Hkv
    out = np.empty((H, D), np.float64)
    for h in range(H):
        g = h // G
        s = (k[:, g, :] @ q[h].astype(np.float64)) * float(np.float32(scale))
        w = np.exp(s - s.max())
        out[h] = (w @ v[:, g, :]) / w.sum()
    return out
