"""Build libtq.so (the HIP kernels and the C ABI of include/tq.h) in-tree.

    python bit_gemv_tq_amd/build.py

(run by path: importing the package itself loads libtq.so) compiles every
``csrc/*.hip`` for gfx950 only with hipcc, in parallel, into objects under
``bit_gemv_tq_amd/_build/`` and links them into ``bit_gemv_tq_amd/libtq.so``.
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
LIB = os.path.join(PKG, "libtq.so")
OBJ_DIR = os.path.join(PKG, "_build")
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-ffp-contract=off",
    "-fvisibility=hidden",
    # Packed fp32 VALU ops stay disabled on this target.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
    "-Wno-unused-command-line-argument",
]


def sources():
    return sorted(glob.glob(os.path.join(PKG, "csrc", "*.hip")))


def _hipcc():
    return os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def build(verbose: bool = False, jobs: int | None = None) -> str:
    os.makedirs(OBJ_DIR, exist_ok=True)
    inc = ["-I", os.path.join(ROOT, "include")]
    pid = os.getpid()

    def compile_one(src):
        obj = os.path.join(OBJ_DIR, os.path.basename(src) + f".{pid}.o")
        cmd = [_hipcc(), *HIPCC_FLAGS, *inc, "-c", src, "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True)
        noise = "is not a recognized feature for this target"
        err = "\n".join(l for l in r.stderr.splitlines() if noise not in l)
        if err.strip():
            print(err, file=sys.stderr, flush=True)
        if r.returncode != 0:
            raise subprocess.CalledProcessError(r.returncode, cmd)
        return obj

    jobs = jobs or max(1, min(8, os.cpu_count() or 1))
    with ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(compile_one, sources()))
    tmp = LIB + ".tmp%d" % pid
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs,
           "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.check_call(cmd)
    os.replace(tmp, LIB)
    for o in objs:
        os.remove(o)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
