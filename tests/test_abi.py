"""C-ABI checks that need no GPU: libtq.so loads, exports every entry point
include/tq.h declares, and rejects every host-detectable bad argument before
any HIP call (so nothing is launched).  Pointers below are fake addresses;
every call here fails validation (or is a documented no-op) before any
pointer could be dereferenced.
"""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tq.h")

OK, NULL, SHAPE, ALIGN, DTYPE, DEVICE, LAUNCH = range(7)


@pytest.fixture(scope="module")
def tq():
    import bit_gemv_tq_amd
    return bit_gemv_tq_amd


def declared_functions():
    text = open(HEADER).read()
    return re.findall(r"TQ_API\s+[\w\s\*]+?\b(tq_\w+)\s*\(", text)


def test_header_declares_the_calls():
    names = declared_functions()
    assert set(names) == {"tq_pack", "tq_act_quant", "tq_gemv", "tq_gemm_small",
                          "tq_gate_up_relu2", "tq_quant_gemv",
                          "tq_quant_gate_up_relu2", "tq_quant_gemv_group",
                          "tq_ternarize", "tq_attn_decode", "tq_rmsnorm_act_quant",
                          "tq_rmsnorm_quant_gemv", "tq_pack3", "tq_gemv3",
                          "tq_stream_read", "tq_attn_decode_noalloc",
                          "tq_status_string"}


def test_library_exports_every_declared_symbol(tq):
    out = subprocess.check_output(["nm", "-D", "--defined-only", tq.LIB_PATH],
                                  text=True)
    exported = {l.split()[-1] for l in out.splitlines() if " T " in l}
    for name in declared_functions():
        assert name in exported, name
        assert getattr(tq.lib, name) is not None
    assert exported == set(declared_functions())   # nothing else leaks
    assert set(tq.EXPORTS) == set(declared_functions())


def test_status_strings(tq):
    for s in range(7):
        assert tq.lib.tq_status_string(s)
    assert b"unknown" in tq.lib.tq_status_string(99)


P = ctypes.c_void_p
A = P(0x10000)          # 64 KiB-aligned fake device address
MIS = P(0x10004)        # 4-aligned, not 16-aligned
ODD = P(0x10001)


def gemv(tq, packed=A, xq=A, xs=A, N=64, K=64, y=A, acc=None):
    return tq.lib.tq_gemv(packed, 0.02, xq, xs, N, K, y, acc, None)


def test_gemv_validation(tq):
    assert gemv(tq, N=6) == SHAPE
    assert gemv(tq, N=-4) == SHAPE
    assert gemv(tq, K=24) == SHAPE
    assert gemv(tq, K=131072 + 16) == SHAPE
    assert gemv(tq, K=-16) == SHAPE
    assert gemv(tq, y=None) == NULL
    assert gemv(tq, xs=None) == NULL
    assert gemv(tq, packed=None) == NULL
    assert gemv(tq, xq=None) == NULL
    assert gemv(tq, packed=MIS) == ALIGN
    assert gemv(tq, xq=MIS) == ALIGN
    assert gemv(tq, y=ODD) == ALIGN
    assert gemv(tq, acc=ODD) == ALIGN
    assert gemv(tq, N=0) == OK                    # empty: no-op


def test_act_quant_validation(tq):
    f = tq.lib.tq_act_quant
    assert f(A, 2, 1, 64, A, A, None) == DTYPE
    assert f(A, 0, 65, 64, A, A, None) == SHAPE
    assert f(A, 0, -1, 64, A, A, None) == SHAPE
    assert f(A, 0, 1, 40, A, A, None) == SHAPE
    assert f(A, 1, 1, 131072 + 16, A, A, None) == SHAPE
    assert f(A, 0, 1, 64, None, A, None) == NULL
    assert f(A, 0, 1, 64, A, None, None) == NULL
    assert f(MIS, 0, 1, 64, A, A, None) == ALIGN
    assert f(A, 0, 1, 64, MIS, A, None) == ALIGN
    assert f(A, 0, 0, 64, A, A, None) == OK


def test_rmsnorm_validation(tq):
    f = tq.lib.tq_rmsnorm_act_quant
    #        x  xt gamma eps     M   K  xq  xs stream
    assert f(A, 2, A, 1e-5, 1, 64, A, A, None) == DTYPE
    assert f(A, 0, A, 0.0, 1, 64, A, A, None) == SHAPE          # eps > 0
    assert f(A, 0, A, -1e-5, 1, 64, A, A, None) == SHAPE
    assert f(A, 0, A, float("inf"), 1, 64, A, A, None) == SHAPE
    assert f(A, 0, A, float("nan"), 1, 64, A, A, None) == SHAPE
    assert f(A, 0, A, 1e-5, 1, 0, A, A, None) == SHAPE          # K > 0
    assert f(A, 0, None, 1e-5, 1, 64, A, A, None) == NULL
    assert f(A, 0, MIS, 1e-5, 1, 64, A, A, None) == ALIGN
    assert f(A, 0, A, 1e-5, 65, 64, A, A, None) == SHAPE
    g = tq.lib.tq_rmsnorm_quant_gemv
    #        x  xt gamma eps  packed  ws   N   K   y  acc  xq  xs stream
    assert g(A, 3, A, 1e-5, A, 0.02, 64, 64, A, None, A, A, None) == DTYPE
    assert g(A, 0, A, 1e-5, A, 0.02, 62, 64, A, None, A, A, None) == SHAPE
    assert g(A, 0, A, 1e-5, A, 0.02, 64, 0, A, None, A, A, None) == SHAPE
    assert g(A, 0, A, 0.0, A, 0.02, 64, 64, A, None, A, A, None) == SHAPE
    assert g(A, 0, None, 1e-5, A, 0.02, 64, 64, A, None, A, A, None) == NULL
    assert g(A, 0, A, 1e-5, None, 0.02, 64, 64, A, None, A, A, None) == NULL
    assert g(A, 0, A, 1e-5, A, 0.02, 64, 64, A, None, None, A, None) == NULL
    assert g(A, 0, MIS, 1e-5, A, 0.02, 64, 64, A, None, A, A, None) == ALIGN
    assert g(A, 0, A, 1e-5, A, 0.02, 64, 64, A, None, MIS, A, None) == ALIGN


def test_pack3_gemv3_validation(tq):
    f = tq.lib.tq_pack3
    assert f(A, 7, 8, A, None) == SHAPE            # K % 16
    assert f(A, -1, 16, A, None) == SHAPE
    assert f(None, 7, 16, A, None) == NULL
    assert f(A, 7, 16, MIS, None) == ALIGN
    assert f(A, 0, 16, A, None) == OK
    g = tq.lib.tq_gemv3
    #        packed ws  xq xs  N   K   y  acc stream
    assert g(A, 0.02, A, A, 7, 8, A, None, None) == SHAPE
    assert g(A, 0.02, A, A, 7, 0, A, None, None) == SHAPE       # K >= 16
    assert g(A, 0.02, A, A, 7, 32784, A, None, None) == SHAPE   # K <= 32768
    assert g(A, 0.02, A, A, -5, 16, A, None, None) == SHAPE
    assert g(None, 0.02, A, A, 7, 16, A, None, None) == NULL
    assert g(A, 0.02, A, A, 7, 16, None, None, None) == NULL
    assert g(A, 0.02, MIS, A, 7, 16, A, None, None) == ALIGN
    assert g(A, 0.02, A, A, 7, 16, A, ODD, None) == ALIGN
    assert g(A, 0.02, A, A, 0, 16, A, None, None) == OK


def test_gemm_small_and_gate_validation(tq):
    g = tq.lib.tq_gemm_small
    assert g(A, 0.02, A, A, 65, 64, 64, A, None, None) == SHAPE
    assert g(A, 0.02, A, A, 4, 62, 64, A, None, None) == SHAPE
    assert g(A, 0.02, A, A, 4, 64, 72, A, None, None) == SHAPE
    assert g(A, 0.02, MIS, A, 4, 64, 64, A, None, None) == ALIGN
    assert g(A, 0.02, A, A, 4, 64, 64, None, None, None) == NULL
    assert g(A, 0.02, A, A, 0, 64, 64, A, None, None) == OK
    h = tq.lib.tq_gate_up_relu2
    assert h(A, 0.02, None, 0.02, A, A, 4, 64, 64, A, None, None, None) == NULL
    assert h(A, 0.02, MIS, 0.02, A, A, 4, 64, 64, A, None, None, None) == ALIGN
    assert h(A, 0.02, A, 0.02, A, A, 4, 64, 64, A, ODD, None, None) == ALIGN
    assert h(A, 0.02, A, 0.02, A, A, 4, 64, 64, A, None, ODD, None) == ALIGN
    assert h(A, 0.02, A, 0.02, A, A, 99, 64, 64, A, None, None, None) == SHAPE


def test_quant_gemv_validation(tq):
    f = tq.lib.tq_quant_gemv
    #       x  xt  packed   ws   N   K   y  acc  xq  xs  ys  stream
    assert f(A, 3, A, 0.02, 64, 64, A, None, A, A, None, None) == DTYPE
    assert f(A, 0, A, 0.02, 62, 64, A, None, A, A, None, None) == SHAPE
    assert f(A, 0, A, 0.02, 64, 40, A, None, A, A, None, None) == SHAPE
    assert f(None, 0, A, 0.02, 64, 64, A, None, A, A, None, None) == NULL
    assert f(A, 0, A, 0.02, 64, 64, A, None, None, A, None, None) == NULL
    assert f(A, 0, A, 0.02, 64, 64, A, None, A, None, None, None) == NULL
    assert f(A, 0, None, 0.02, 64, 64, A, None, A, A, None, None) == NULL
    assert f(A, 0, A, 0.02, 64, 64, None, None, A, A, None, None) == NULL
    assert f(MIS, 0, A, 0.02, 64, 64, A, None, A, A, None, None) == ALIGN
    assert f(A, 0, A, 0.02, 64, 64, A, None, MIS, A, None, None) == ALIGN
    assert f(A, 0, A, 0.02, 64, 64, A, None, A, A, ODD, None) == ALIGN
    g = tq.lib.tq_quant_gate_up_relu2
    assert g(A, 1, A, 0.02, None, 0.02, 64, 64, A, None, None, A, A, None,
             None) == NULL
    assert g(A, 1, A, 0.02, MIS, 0.02, 64, 64, A, None, None, A, A, None,
             None) == ALIGN


def test_quant_gemv_group_validation(tq):
    f = tq.lib.tq_quant_gemv_group
    VP = ctypes.c_void_p * 3
    packed = VP(0x10000, 0x20000, 0x30000)
    scale = (ctypes.c_float * 3)(0.02, 0.03, 0.04)
    ys = VP(0x40000, 0x50000, 0x60000)

    def call(count=3, xt=1, Ns=(64, 16, 16), K=64, packed=packed, ys=ys,
             acc=None, x=A, xq=A, xs=A, ysc=None):
        n = (ctypes.c_int64 * 3)(*Ns)
        c = lambda a: None if a is None else ctypes.cast(a, ctypes.c_void_p)
        return f(x, xt, count, c(packed), c(scale), c(n), K, c(ys), c(acc),
                 xq, xs, ysc, None)
    assert call(count=0) == SHAPE
    assert call(count=5) == SHAPE
    assert call(xt=2) == DTYPE
    assert call(Ns=(64, 18, 16)) == SHAPE
    assert call(K=40) == SHAPE
    assert call(packed=None) == NULL
    assert call(ys=None) == NULL
    assert call(ys=VP(0x40000, None, 0x60000)) == NULL
    assert call(packed=VP(0x10000, 0x20004, 0x30000)) == ALIGN
    assert call(acc=VP(None, 0x70001, None)) == ALIGN
    assert call(x=MIS) == ALIGN
    assert call(xq=None) == NULL


def test_ternarize_validation(tq):
    f = tq.lib.tq_ternarize
    assert f(A, 6, 16, A, A, A, None) == SHAPE
    assert f(A, 8, 24, A, A, A, None) == SHAPE
    assert f(A, -4, 16, A, A, A, None) == SHAPE
    assert f(A, 1 << 20, 1 << 12, A, A, A, None) == SHAPE     # N*K > 2^31 - 1
    assert f(A, 8, 16, A, None, A, None) == NULL
    assert f(A, 8, 16, A, A, None, None) == NULL
    assert f(None, 8, 16, A, A, A, None) == NULL
    assert f(A, 8, 16, None, A, A, None) == NULL
    assert f(MIS, 8, 16, A, A, A, None) == ALIGN
    assert f(A, 8, 16, MIS, A, A, None) == ALIGN
    assert f(A, 8, 16, A, ODD, A, None) == ALIGN
    assert f(A, 8, 16, A, A, P(0x10004), None) == ALIGN


def test_attn_decode_validation(tq):
    f = tq.lib.tq_attn_decode
    W = tq.attn_workspace_bytes(20, 128, 16)
    #        q  k  v   H  Hkv  D    L   scale  out ws  bytes stream
    assert f(A, A, A, 20, 3, 128, 16, 0.1, A, A, W, None) == SHAPE      # H % Hkv
    assert f(A, A, A, 48, 4, 128, 16, 0.1, A, A, W, None) == SHAPE      # group 12
    assert f(A, A, A, 20, 5, 96, 16, 0.1, A, A, W, None) == SHAPE       # D
    assert f(A, A, A, 20, 5, 128, 0, 0.1, A, A, W, None) == SHAPE       # L = 0
    assert f(A, A, A, 20, 5, 128, 131073, 0.1, A, A, 1 << 40, None) == SHAPE
    assert f(A, A, A, 20, 5, 128, 16, 0.1, A, A, W - 1, None) == SHAPE  # workspace
    assert f(A, A, A, 20, 5, 128, 64 * 1000 + 1, 0.1, A, A,
             tq.attn_workspace_bytes(20, 128, 64 * 1000), None) == SHAPE
    assert f(None, A, A, 20, 5, 128, 16, 0.1, A, A, W, None) == NULL
    assert f(A, A, A, 20, 5, 128, 16, 0.1, A, None, W, None) == NULL
    assert f(MIS, A, A, 20, 5, 128, 16, 0.1, A, A, W, None) == ALIGN
    assert f(A, MIS, A, 20, 5, 128, 16, 0.1, A, A, W, None) == ALIGN
    assert f(A, A, A, 20, 5, 128, 16, 0.1, ODD, A, W, None) == ALIGN
    assert f(A, A, A, 20, 5, 128, 16, 0.1, A, P(0x10008), W, None) == ALIGN


def test_attn_decode_noalloc_validation(tq):
    f = tq.lib.tq_attn_decode_noalloc
    #        q  k  v   H  Hkv  D    L   scale  out stream
    assert f(A, A, A, 72, 9, 128, 16, 0.1, A, None) == SHAPE      # H > 64
    assert f(A, A, A, 128, 16, 64, 16, 0.1, A, None) == SHAPE     # H > 64
    assert f(A, A, A, 20, 3, 128, 16, 0.1, A, None) == SHAPE      # H % Hkv
    assert f(A, A, A, 48, 4, 128, 16, 0.1, A, None) == SHAPE      # group 12
    assert f(A, A, A, 20, 5, 96, 16, 0.1, A, None) == SHAPE       # D
    assert f(A, A, A, 20, 5, 128, 0, 0.1, A, None) == SHAPE       # L = 0
    assert f(A, A, A, 20, 5, 128, 131073, 0.1, A, None) == SHAPE
    assert f(None, A, A, 20, 5, 128, 16, 0.1, A, None) == NULL
    assert f(A, A, A, 20, 5, 128, 16, 0.1, None, None) == NULL
    assert f(MIS, A, A, 20, 5, 128, 16, 0.1, A, None) == ALIGN
    assert f(A, A, MIS, 20, 5, 128, 16, 0.1, A, None) == ALIGN
    assert f(A, A, A, 20, 5, 128, 16, 0.1, ODD, None) == ALIGN


def test_attn_noalloc_scratch_size():
    # TQ_ATTN_NOALLOC_SCRATCH_BYTES: 64 heads x 64 chunks x (128 + 4) floats
    text = open(HEADER).read()
    assert "#define TQ_ATTN_NOALLOC_MAX_H 64" in text
    assert 64 * 64 * 132 * 4 == 2162688


def test_attn_workspace_size(tq):
    # TQ_ATTN_WORKSPACE_BYTES: H x ceil(L / 64) fp32 chunk rows of D + 4
    assert tq.attn_workspace_bytes(20, 128, 2048) == 20 * 32 * 132 * 4
    assert tq.attn_workspace_bytes(1, 64, 1) == 68 * 4
    assert tq.attn_workspace_bytes(20, 128, 2049) == 20 * 33 * 132 * 4


def test_pack_validation(tq):
    f = tq.lib.tq_pack
    assert f(A, 5, 16, A, None) == SHAPE
    assert f(A, 8, 8, A, None) == SHAPE
    assert f(None, 8, 16, A, None) == NULL
    assert f(A, 8, 16, MIS, None) == ALIGN
    assert f(A, 0, 16, A, None) == OK


def _no_gpu():
    try:
        import torch
        return not torch.cuda.is_available()
    except Exception:
        return True


@pytest.mark.skipif(not _no_gpu(), reason="checks the no-device path")
def test_stream_read_validation(tq):
    f = tq.lib.tq_stream_read
    #        buf  bytes sink words stream
    assert f(A, 24, A, 8, None) == SHAPE       # bytes % 16
    assert f(A, -16, A, 8, None) == SHAPE
    assert f(A, 64, A, 0, None) == SHAPE       # sink_words >= 1
    assert f(None, 64, A, 8, None) == NULL
    assert f(A, 64, None, 8, None) == NULL
    assert f(MIS, 64, A, 8, None) == ALIGN
    assert f(A, 64, MIS, 8, None) == ALIGN
    assert f(A, 0, A, 8, None) == OK           # empty: no-op


def test_no_device_is_reported(tq):
    # Valid arguments on a machine with no GPU: TQ_ERR_DEVICE, nothing runs.
    assert gemv(tq) == DEVICE
    assert tq.lib.tq_act_quant(A, 0, 1, 64, A, A, None) == DEVICE
    assert tq.lib.tq_pack(A, 8, 16, A, None) == DEVICE
    assert tq.lib.tq_ternarize(A, 8, 16, A, A, A, None) == DEVICE
    assert tq.lib.tq_rmsnorm_act_quant(A, 0, A, 1e-5, 1, 64, A, A, None) == DEVICE
    assert tq.lib.tq_pack3(A, 7, 16, A, None) == DEVICE
    assert tq.lib.tq_gemv3(A, 0.02, A, A, 7, 16, A, None, None) == DEVICE
    assert tq.lib.tq_stream_read(A, 64, A, 8, None) == DEVICE
    assert tq.lib.tq_rmsnorm_quant_gemv(A, 0, A, 1e-5, A, 0.02, 64, 64, A, None, A, A,
                                        None) == DEVICE
    assert tq.lib.tq_attn_decode(A, A, A, 20, 5, 128, 16, 0.1, A, A,
                                 tq.attn_workspace_bytes(20, 128, 16), None) == DEVICE
    assert tq.lib.tq_gemm_small(A, 0.02, A, A, 4, 64, 64, A, None, None) == DEVICE
    assert tq.lib.tq_quant_gemv(A, 0, A, 0.02, 64, 64, A, None, A, A, None,
                                None) == DEVICE
    one = (ctypes.c_void_p * 1)(0x10000)
    assert tq.lib.tq_quant_gemv_group(
        A, 0, 1, ctypes.cast(one, ctypes.c_void_p),
        ctypes.cast((ctypes.c_float * 1)(0.02), ctypes.c_void_p),
        ctypes.cast((ctypes.c_int64 * 1)(64), ctypes.c_void_p), 64,
        ctypes.cast(one, ctypes.c_void_p), None, A, A, None, None) == DEVICE


def test_binding_rejects_host_tensors(tq):
    import torch
    w = torch.zeros(8, 16, dtype=torch.int8)
    with pytest.raises(ValueError):
        tq.tq_pack(w)
    with pytest.raises(TypeError):
        tq.tq_pack(w.to(torch.int32))
    with pytest.raises(TypeError):
        tq.tq_act_quant(torch.zeros(16, dtype=torch.float16))
