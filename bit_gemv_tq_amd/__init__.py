"""Python binding of libtq, the gfx950 ternary GEMV library (include/tq.h).

Argument marshalling only: every step of the computation runs in the HIP
kernels of ``libtq.so``.  PyTorch provides device memory and the current
stream; outputs that are not passed in are allocated with ``torch.empty`` on
the input's device.  There is no CPU fallback: importing this package fails
if ``libtq.so`` has not been built (``python bit_gemv_tq_amd/build.py``),
and every call raises ``TQError`` on a non-OK status.

Conventions (weights, packing, activation quantization and rescale) are the
ones documented in include/tq.h.
"""
from __future__ import annotations

import ctypes
import math
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libtq.so")

TQ_BF16 = 0
TQ_F32 = 1
TQ_MAX_K = 131072
TQ_MAX_M = 64

STATUS = {0: "TQ_OK", 1: "TQ_ERR_NULL", 2: "TQ_ERR_SHAPE", 3: "TQ_ERR_ALIGN",
          4: "TQ_ERR_DTYPE", 5: "TQ_ERR_DEVICE", 6: "TQ_ERR_LAUNCH"}

EXPORTS = ("tq_pack", "tq_act_quant", "tq_gemv", "tq_gemm_small",
           "tq_gate_up_relu2", "tq_quant_gemv", "tq_quant_gate_up_relu2",
           "tq_quant_gemv_group", "tq_ternarize", "tq_attn_decode",
           "tq_rmsnorm_act_quant", "tq_rmsnorm_quant_gemv", "tq_pack3", "tq_gemv3",
           "tq_stream_read", "tq_attn_decode_noalloc", "tq_status_string")


class TQError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        text = lib.tq_status_string(status).decode()
        super().__init__(f"{fn}: {STATUS.get(status, status)} ({text})")


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build the HIP library first with "
            "`python bit_gemv_tq_amd/build.py` (hipcc, gfx950)")
    L = ctypes.CDLL(LIB_PATH)
    p, i64, f32, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_float, ctypes.c_int
    sigs = {
        "tq_pack": [p, i64, i64, p, p],
        "tq_act_quant": [p, i32, i64, i64, p, p, p],
        "tq_gemv": [p, f32, p, p, i64, i64, p, p, p],
        "tq_gemm_small": [p, f32, p, p, i64, i64, i64, p, p, p],
        "tq_gate_up_relu2": [p, f32, p, f32, p, p, i64, i64, i64, p, p, p, p],
        "tq_quant_gemv": [p, i32, p, f32, i64, i64, p, p, p, p, p, p],
        "tq_quant_gate_up_relu2": [p, i32, p, f32, p, f32, i64, i64, p, p, p,
                                   p, p, p, p],
        # host arrays: packed**, w_scale*, N*, y**, acc** (ctypes arrays)
        "tq_quant_gemv_group": [p, i32, i32, p, p, p, i64, p, p, p, p, p, p],
        "tq_ternarize": [p, i64, i64, p, p, p, p],
        "tq_attn_decode": [p, p, p, i64, i64, i64, i64, f32, p, p, ctypes.c_size_t, p],
        "tq_attn_decode_noalloc": [p, p, p, i64, i64, i64, i64, f32, p, p],
        "tq_rmsnorm_act_quant": [p, i32, p, f32, i64, i64, p, p, p],
        "tq_pack3": [p, i64, i64, p, p],
        "tq_gemv3": [p, f32, p, p, i64, i64, p, p, p],
        "tq_stream_read": [p, i64, p, i64, p],
        "tq_rmsnorm_quant_gemv": [p, i32, p, f32, p, f32, i64, i64, p, p, p, p, p],
    }
    for name, args in sigs.items():
        fn = getattr(L, name)
        fn.argtypes = args
        fn.restype = ctypes.c_int
    L.tq_status_string.argtypes = [ctypes.c_int]
    L.tq_status_string.restype = ctypes.c_char_p
    return L


lib = _load()


# --------------------------------------------------------------------------
# marshalling helpers
# --------------------------------------------------------------------------
def _torch():
    import torch
    return torch


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _need(t, name, dtype, device=None):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a GPU device, got {t.device}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _check(fn, status):
    if status != 0:
        raise TQError(fn, status)


def _out(t, name, shape, dtype, device):
    torch = _torch()
    if t is None:
        return torch.empty(shape, dtype=dtype, device=device)
    _need(t, name, dtype, device)
    if t.numel() != math.prod(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, need {tuple(shape)}")
    return t


# --------------------------------------------------------------------------
# the five calls
# --------------------------------------------------------------------------
def tq_pack(w, packed=None, stream=None):
    """int8 ternary weights [N, K] -> packed uint8 [N/4, K]."""
    torch = _torch()
    _need(w, "w", torch.int8)
    N, K = w.shape
    packed = _out(packed, "packed", (N // 4, K), torch.uint8, w.device)
    _check("tq_pack", lib.tq_pack(_ptr(w), N, K, _ptr(packed), _stream(stream)))
    return packed


def tq_pack3(w, packed=None, stream=None):
    """int8 ternary weights [N, K] -> uint8 [ceil(N/5), K], five weights per
    byte (the denser layout of tq_gemv3)."""
    torch = _torch()
    _need(w, "w", torch.int8)
    N, K = w.shape
    packed = _out(packed, "packed", ((N + 4) // 5, K), torch.uint8, w.device)
    _check("tq_pack3", lib.tq_pack3(_ptr(w), N, K, _ptr(packed), _stream(stream)))
    return packed


def tq_gemv3(packed, w_scale, xq, x_scale, N, y=None, acc=None, stream=None):
    """tq_gemv on the five-per-byte layout (packed [ceil(N/5), K]); returns y."""
    torch = _torch()
    _need(packed, "packed", torch.uint8)
    dev = packed.device
    K = packed.shape[1]
    if packed.shape[0] != (N + 4) // 5:
        raise ValueError(f"packed has {packed.shape[0]} rows, need ceil({N}/5)")
    _need(xq, "xq", torch.int8, dev)
    _need(x_scale, "x_scale", torch.float32, dev)
    y = _out(y, "y", (N,), torch.float32, dev)
    if acc is not None:
        acc = _out(acc, "acc", (N,), torch.int32, dev)
    _check("tq_gemv3", lib.tq_gemv3(_ptr(packed), float(w_scale), _ptr(xq),
                                    _ptr(x_scale), N, K, _ptr(y), _ptr(acc),
                                    _stream(stream)))
    return y


def tq_stream_read(buf, sink=None, stream=None):
    """Read the whole contiguous device tensor `buf` (byte size a multiple
    of 16) with the GEMV's access pattern and nothing else (the measured read
    ceiling).  Returns `sink`, uint32 [words, 4]: block b's word is the XOR
    of the 16-byte words it read (unused words are zeroed when the sink is
    allocated here)."""
    torch = _torch()
    if not isinstance(buf, torch.Tensor) or buf.device.type != "cuda":
        raise ValueError("buf must be a GPU tensor")
    if not buf.is_contiguous():
        raise ValueError("buf must be contiguous")
    nbytes = buf.numel() * buf.element_size()
    if sink is None:
        sink = torch.zeros(4096, 4, dtype=torch.int32, device=buf.device)
    _need(sink, "sink", torch.int32, buf.device)
    if sink.dim() != 2 or sink.shape[1] != 4:
        raise ValueError("sink must be int32 [words, 4]")
    _check("tq_stream_read", lib.tq_stream_read(_ptr(buf), nbytes, _ptr(sink),
                                                sink.shape[0], _stream(stream)))
    return sink


def tq_act_quant(x, xq=None, x_scale=None, stream=None):
    """Per-row absmax int8 quantization of bf16 or fp32 x [M, K] (or [K]).
    Returns (xq int8 [M, K], x_scale fp32 [M])."""
    torch = _torch()
    if x.dtype == torch.bfloat16:
        xt = TQ_BF16
    elif x.dtype == torch.float32:
        xt = TQ_F32
    else:
        raise TypeError(f"x must be bfloat16 or float32, got {x.dtype}")
    _need(x, "x", x.dtype)
    x2 = x.reshape(1, -1) if x.dim() == 1 else x
    M, K = x2.shape
    xq = _out(xq, "xq", (M, K), torch.int8, x.device)
    x_scale = _out(x_scale, "x_scale", (M,), torch.float32, x.device)
    _check("tq_act_quant", lib.tq_act_quant(_ptr(x2), xt, M, K, _ptr(xq),
                                            _ptr(x_scale), _stream(stream)))
    return xq, x_scale


def tq_gemv(packed, w_scale, xq, x_scale, y=None, acc=None, stream=None):
    """y[n] = (float)sum_k w[n,k] q[k] * (w_scale * x_scale[0]) at M = 1."""
    torch = _torch()
    _need(packed, "packed", torch.uint8)
    dev = packed.device
    _need(xq, "xq", torch.int8, dev)
    _need(x_scale, "x_scale", torch.float32, dev)
    N, K = packed.shape[0] * 4, packed.shape[1]
    if xq.numel() != K:
        raise ValueError(f"xq has {xq.numel()} elements, need K={K}")
    y = _out(y, "y", (N,), torch.float32, dev)
    if acc is not None:
        acc = _out(acc, "acc", (N,), torch.int32, dev)
    _check("tq_gemv", lib.tq_gemv(_ptr(packed), float(w_scale), _ptr(xq),
                                  _ptr(x_scale), N, K, _ptr(y), _ptr(acc),
                                  _stream(stream)))
    return y


def tq_gemm_small(packed, w_scale, xq, x_scale, y=None, acc=None, stream=None):
    """y[m,n] for a small batch xq [M, K] (M <= 64): int8 matrix cores, or
    the vector ALU for M = 2 (K <= 16384), where that measured faster."""
    torch = _torch()
    _need(packed, "packed", torch.uint8)
    dev = packed.device
    _need(xq, "xq", torch.int8, dev)
    _need(x_scale, "x_scale", torch.float32, dev)
    N, K = packed.shape[0] * 4, packed.shape[1]
    xq2 = xq.reshape(1, -1) if xq.dim() == 1 else xq
    M = xq2.shape[0]
    if xq2.shape[1] != K:
        raise ValueError(f"xq has K={xq2.shape[1]}, packed has K={K}")
    y = _out(y, "y", (M, N), torch.float32, dev)
    if acc is not None:
        acc = _out(acc, "acc", (M, N), torch.int32, dev)
    _check("tq_gemm_small", lib.tq_gemm_small(
        _ptr(packed), float(w_scale), _ptr(xq2), _ptr(x_scale), M, N, K,
        _ptr(y), _ptr(acc), _stream(stream)))
    return y


def tq_gate_up_relu2(packed_gate, s_gate, packed_up, s_up, xq, x_scale,
                     h=None, acc_gate=None, acc_up=None, stream=None):
    """h = relu(g)^2 * u with g, u the gate and up projections of xq [M, K]."""
    torch = _torch()
    _need(packed_gate, "packed_gate", torch.uint8)
    dev = packed_gate.device
    _need(packed_up, "packed_up", torch.uint8, dev)
    if packed_up.shape != packed_gate.shape:
        raise ValueError("packed_gate and packed_up shapes differ")
    _need(xq, "xq", torch.int8, dev)
    _need(x_scale, "x_scale", torch.float32, dev)
    N, K = packed_gate.shape[0] * 4, packed_gate.shape[1]
    xq2 = xq.reshape(1, -1) if xq.dim() == 1 else xq
    M = xq2.shape[0]
    if xq2.shape[1] != K:
        raise ValueError(f"xq has K={xq2.shape[1]}, packed has K={K}")
    h = _out(h, "h", (M, N), torch.float32, dev)
    if acc_gate is not None:
        acc_gate = _out(acc_gate, "acc_gate", (M, N), torch.int32, dev)
    if acc_up is not None:
        acc_up = _out(acc_up, "acc_up", (M, N), torch.int32, dev)
    _check("tq_gate_up_relu2", lib.tq_gate_up_relu2(
        _ptr(packed_gate), float(s_gate), _ptr(packed_up), float(s_up),
        _ptr(xq2), _ptr(x_scale), M, N, K, _ptr(h), _ptr(acc_gate),
        _ptr(acc_up), _stream(stream)))
    return h


def _raw_row(x):
    torch = _torch()
    if x.dtype == torch.bfloat16:
        xt = TQ_BF16
    elif x.dtype == torch.float32:
        xt = TQ_F32
    else:
        raise TypeError(f"x must be bfloat16 or float32, got {x.dtype}")
    _need(x, "x", x.dtype)
    return xt


def tq_quant_gemv(x, packed, w_scale, y=None, acc=None, xq=None, x_scale=None,
                  y_scale=None, stream=None):
    """act_quant + gemv at M = 1 in one launch.  x: bf16/fp32 [K].  Returns
    y; the quantized row and its scale land in xq / x_scale (allocated when
    not given).  y_scale: optional fp32 [1] used in the rescale instead of
    the row's own s_x."""
    torch = _torch()
    xt = _raw_row(x)
    _need(packed, "packed", torch.uint8, x.device)
    dev = packed.device
    N, K = packed.shape[0] * 4, packed.shape[1]
    if x.numel() != K:
        raise ValueError(f"x has {x.numel()} elements, need K={K}")
    y = _out(y, "y", (N,), torch.float32, dev)
    if acc is not None:
        acc = _out(acc, "acc", (N,), torch.int32, dev)
    xq = _out(xq, "xq", (K,), torch.int8, dev)
    x_scale = _out(x_scale, "x_scale", (1,), torch.float32, dev)
    if y_scale is not None:
        _need(y_scale, "y_scale", torch.float32, dev)
    _check("tq_quant_gemv", lib.tq_quant_gemv(
        _ptr(x), xt, _ptr(packed), float(w_scale), N, K, _ptr(y), _ptr(acc),
        _ptr(xq), _ptr(x_scale), _ptr(y_scale), _stream(stream)))
    return y


def _gamma(gamma, x):
    if gamma.dtype != x.dtype:
        raise TypeError(f"gamma must have the dtype of x ({x.dtype}), got {gamma.dtype}")
    _need(gamma, "gamma", x.dtype, x.device)
    return gamma


def tq_rmsnorm_act_quant(x, gamma, eps=1e-5, xq=None, x_scale=None, stream=None):
    """Sub-layer RMSNorm folded into per-row absmax quantization: x bf16 or
    fp32 [M, K] (or [K]), gamma [K] of the same dtype.  Returns (xq int8
    [M, K], x_scale fp32 [M]) with xq * x_scale ~ RMSNorm(x) * gamma."""
    torch = _torch()
    xt = _raw_row(x)
    x2 = x.reshape(1, -1) if x.dim() == 1 else x
    M, K = x2.shape
    _gamma(gamma, x)
    if gamma.numel() != K:
        raise ValueError(f"gamma has {gamma.numel()} elements, need K={K}")
    xq = _out(xq, "xq", (M, K), torch.int8, x.device)
    x_scale = _out(x_scale, "x_scale", (M,), torch.float32, x.device)
    _check("tq_rmsnorm_act_quant", lib.tq_rmsnorm_act_quant(
        _ptr(x2), xt, _ptr(gamma), float(eps), M, K, _ptr(xq), _ptr(x_scale),
        _stream(stream)))
    return xq, x_scale


def tq_rmsnorm_quant_gemv(x, gamma, packed, w_scale, eps=1e-5, y=None, acc=None,
                          xq=None, x_scale=None, stream=None):
    """RMSNorm + act_quant + gemv at M = 1 in one launch.  x: bf16/fp32 [K],
    gamma [K] of the same dtype.  Returns y; the quantized row and its scale
    land in xq / x_scale (allocated when not given)."""
    torch = _torch()
    xt = _raw_row(x)
    _gamma(gamma, x)
    _need(packed, "packed", torch.uint8, x.device)
    dev = packed.device
    N, K = packed.shape[0] * 4, packed.shape[1]
    if x.numel() != K or gamma.numel() != K:
        raise ValueError(f"x and gamma need K={K} elements")
    y = _out(y, "y", (N,), torch.float32, dev)
    if acc is not None:
        acc = _out(acc, "acc", (N,), torch.int32, dev)
    xq = _out(xq, "xq", (K,), torch.int8, dev)
    x_scale = _out(x_scale, "x_scale", (1,), torch.float32, dev)
    _check("tq_rmsnorm_quant_gemv", lib.tq_rmsnorm_quant_gemv(
        _ptr(x), xt, _ptr(gamma), float(eps), _ptr(packed), float(w_scale), N, K,
        _ptr(y), _ptr(acc), _ptr(xq), _ptr(x_scale), _stream(stream)))
    return y


def tq_quant_gemv_group(x, packed, w_scale, y=None, acc=None, xq=None,
                        x_scale=None, y_scale=None, stream=None):
    """tq_quant_gemv over several matrices sharing x, in one launch.
    packed / w_scale: lists (1..4 entries); y / acc: optional lists of
    outputs (entries may be None in acc).  Returns the list of y."""
    torch = _torch()
    xt = _raw_row(x)
    count = len(packed)
    if not 1 <= count <= 4 or len(w_scale) != count:
        raise ValueError("need 1..4 matrices and one scale each")
    dev = packed[0].device
    K = packed[0].shape[1]
    for P in packed:
        _need(P, "packed", torch.uint8, x.device)
        if P.shape[1] != K:
            raise ValueError("all matrices must share K")
    if x.numel() != K:
        raise ValueError(f"x has {x.numel()} elements, need K={K}")
    Ns = [P.shape[0] * 4 for P in packed]
    y = [None] * count if y is None else list(y)
    y = [_out(t, "y", (n,), torch.float32, dev) for t, n in zip(y, Ns)]
    if acc is not None:
        acc = [None if t is None else _out(t, "acc", (n,), torch.int32, dev)
               for t, n in zip(acc, Ns)]
    xq = _out(xq, "xq", (K,), torch.int8, dev)
    x_scale = _out(x_scale, "x_scale", (1,), torch.float32, dev)
    if y_scale is not None:
        _need(y_scale, "y_scale", torch.float32, dev)
    VP = ctypes.c_void_p * count
    addr = lambda t: None if t is None else t.data_ptr()
    c_packed = VP(*[addr(P) for P in packed])
    c_scale = (ctypes.c_float * count)(*[float(s) for s in w_scale])
    c_n = (ctypes.c_int64 * count)(*Ns)
    c_y = VP(*[addr(t) for t in y])
    c_acc = None if acc is None else VP(*[addr(t) for t in acc])
    _check("tq_quant_gemv_group", lib.tq_quant_gemv_group(
        _ptr(x), xt, count, ctypes.cast(c_packed, ctypes.c_void_p),
        ctypes.cast(c_scale, ctypes.c_void_p), ctypes.cast(c_n, ctypes.c_void_p),
        K, ctypes.cast(c_y, ctypes.c_void_p),
        None if c_acc is None else ctypes.cast(c_acc, ctypes.c_void_p),
        _ptr(xq), _ptr(x_scale), _ptr(y_scale), _stream(stream)))
    return y


TQ_TERNARIZE_WORKSPACE_BYTES = 4096
_ws_cache = {}


def tq_ternarize(w, packed=None, w_scale=None, workspace=None, stream=None):
    """bf16 weights [N, K] -> (packed uint8 [N/4, K], w_scale fp32 [1]) by
    the absmean rule (exact mean, one rounding).  The workspace (device,
    >= TQ_TERNARIZE_WORKSPACE_BYTES) is cached per device when not given;
    calls that may overlap on different streams must pass their own."""
    torch = _torch()
    if w.dtype != torch.bfloat16:
        raise TypeError(f"w must be bfloat16, got {w.dtype}")
    _need(w, "w", torch.bfloat16, w.device)
    if w.dim() != 2:
        raise ValueError("w must be [N, K]")
    N, K = w.shape
    dev = w.device
    packed = _out(packed, "packed", (N // 4, K), torch.uint8, dev)
    w_scale = _out(w_scale, "w_scale", (1,), torch.float32, dev)
    if workspace is None:
        key = (dev.type, dev.index)
        workspace = _ws_cache.get(key)
        if workspace is None:
            workspace = torch.empty(TQ_TERNARIZE_WORKSPACE_BYTES, dtype=torch.uint8,
                                    device=dev)
            _ws_cache[key] = workspace
    elif workspace.numel() * workspace.element_size() < TQ_TERNARIZE_WORKSPACE_BYTES:
        raise ValueError("workspace too small")
    _check("tq_ternarize", lib.tq_ternarize(_ptr(w), N, K, _ptr(packed), _ptr(w_scale),
                                            _ptr(workspace), _stream(stream)))
    return packed, w_scale


TQ_ATTN_MAX_L = 131072


def attn_workspace_bytes(H: int, D: int, L: int) -> int:
    """TQ_ATTN_WORKSPACE_BYTES(H, D, L): per-chunk partial results."""
    return H * ((L + 63) // 64) * (D + 4) * 4


_attn_ws_cache = {}


def attn_workspace(H: int, D: int, L: int, device):
    """A workspace for tq_attn_decode calls with these H, D and any length up to L."""
    torch = _torch()
    return torch.empty(attn_workspace_bytes(H, D, L), dtype=torch.uint8, device=device)


def tq_attn_decode(q, k_cache, v_cache, scale=None, out=None, workspace=None,
                   stream=None):
    """Attention of one query token: q fp32 [H, D], k/v bf16 [L, Hkv, D] ->
    out fp32 [H, D] (fp32 within chunks, fp64 merge, one rounding).  scale
    defaults to 1/sqrt(D) rounded to fp32.  Without a workspace, one per
    device is kept and grown as needed (calls that may overlap on different
    streams must pass their own)."""
    torch = _torch()
    _need(q, "q", torch.float32)
    dev = q.device
    _need(k_cache, "k_cache", torch.bfloat16, dev)
    _need(v_cache, "v_cache", torch.bfloat16, dev)
    if q.dim() != 2 or k_cache.dim() != 3 or v_cache.shape != k_cache.shape:
        raise ValueError("need q [H, D] and k/v [L, Hkv, D]")
    H, D = q.shape
    L, Hkv, Dk = k_cache.shape
    if Dk != D:
        raise ValueError("head dims differ")
    if scale is None:
        scale = ctypes.c_float(1.0 / math.sqrt(D)).value
    out = _out(out, "out", (H, D), torch.float32, dev)
    need = attn_workspace_bytes(H, D, L)
    if workspace is None:
        key = (dev.type, dev.index)
        workspace = _attn_ws_cache.get(key)
        if workspace is None or workspace.numel() < need:
            workspace = attn_workspace(H, D, L, dev)
            _attn_ws_cache[key] = workspace
    elif workspace.numel() * workspace.element_size() < need:
        raise ValueError("workspace too small")
    _check("tq_attn_decode", lib.tq_attn_decode(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), H, Hkv, D, L, float(scale),
        _ptr(out), _ptr(workspace), workspace.numel() * workspace.element_size(),
        _stream(stream)))
    return out


TQ_ATTN_NOALLOC_MAX_H = 64


def tq_attn_decode_noalloc(q, k_cache, v_cache, scale=None, out=None, stream=None):
    """tq_attn_decode with the library's fixed per-GPU scratch instead of a
    workspace (H <= 64): the call allocates nothing on the device when `out`
    is passed.  Calls that may overlap in time on one GPU must not be
    issued (they share that scratch)."""
    torch = _torch()
    _need(q, "q", torch.float32)
    dev = q.device
    _need(k_cache, "k_cache", torch.bfloat16, dev)
    _need(v_cache, "v_cache", torch.bfloat16, dev)
    if q.dim() != 2 or k_cache.dim() != 3 or v_cache.shape != k_cache.shape:
        raise ValueError("need q [H, D] and k/v [L, Hkv, D]")
    H, D = q.shape
    L, Hkv, Dk = k_cache.shape
    if Dk != D:
        raise ValueError("head dims differ")
    if scale is None:
        scale = ctypes.c_float(1.0 / math.sqrt(D)).value
    out = _out(out, "out", (H, D), torch.float32, dev)
    _check("tq_attn_decode_noalloc", lib.tq_attn_decode_noalloc(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), H, Hkv, D, L, float(scale),
        _ptr(out), _stream(stream)))
    return out


def tq_quant_gate_up_relu2(x, packed_gate, s_gate, packed_up, s_up, h=None,
                           acc_gate=None, acc_up=None, xq=None, x_scale=None,
                           y_scale=None, stream=None):
    """act_quant + gate/up + relu^2 at M = 1 in one launch.  Returns h."""
    torch = _torch()
    xt = _raw_row(x)
    _need(packed_gate, "packed_gate", torch.uint8, x.device)
    dev = packed_gate.device
    _need(packed_up, "packed_up", torch.uint8, dev)
    if packed_up.shape != packed_gate.shape:
        raise ValueError("packed_gate and packed_up shapes differ")
    N, K = packed_gate.shape[0] * 4, packed_gate.shape[1]
    if x.numel() != K:
        raise ValueError(f"x has {x.numel()} elements, need K={K}")
    h = _out(h, "h", (N,), torch.float32, dev)
    if acc_gate is not None:
        acc_gate = _out(acc_gate, "acc_gate", (N,), torch.int32, dev)
    if acc_up is not None:
        acc_up = _out(acc_up, "acc_up", (N,), torch.int32, dev)
    xq = _out(xq, "xq", (K,), torch.int8, dev)
    x_scale = _out(x_scale, "x_scale", (1,), torch.float32, dev)
    if y_scale is not None:
        _need(y_scale, "y_scale", torch.float32, dev)
    _check("tq_quant_gate_up_relu2", lib.tq_quant_gate_up_relu2(
        _ptr(x), xt, _ptr(packed_gate), float(s_gate), _ptr(packed_up),
        float(s_up), N, K, _ptr(h), _ptr(acc_gate), _ptr(acc_up), _ptr(xq),
        _ptr(x_scale), _ptr(y_scale), _stream(stream)))
    return h
