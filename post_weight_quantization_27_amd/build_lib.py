"""Build libpwq.so (the HIP kernels and the C ABI) for gfx950 with hipcc, in-tree.

Every source is compiled to an object under _build/ in parallel, then linked into
post_weight_quantization_27_amd/libpwq.so.  No fast-math flags: the quantizer relies on
IEEE float32 division and square root.  Packed-FP32 instruction selection is disabled.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libpwq.so")

SOURCES = ["hessian.hip", "chol.hip", "gptq.hip", "rtn.hip", "mse.hip", "w4a16.hip", "awq.hip", "pwq_api.hip"]
ARCH = os.environ.get("PWQ_OFFLOAD_ARCH", "gfx950")
CFLAGS = [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          # the GPTQ column loop is unrolled in full (static register indices); its body is
          # larger than LLVM's default limit for pragma-requested unrolling
          "-mllvm", "-pragma-unroll-threshold=1000000",
          "-I", os.path.join(ROOT, "include")]


def _hipcc() -> str:
    for c in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


def _run(cmd):
    p = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in p.stdout.splitlines() if "packed-fp32-ops" not in l)
    if p.returncode != 0:
        raise RuntimeError(f"command failed ({p.returncode}): {' '.join(cmd)}\n{out}")
    return out


def build(verbose: bool = False, jobs: int = 0) -> str:
    """Compile every HIP source and link libpwq.so; returns the library path."""
    hipcc = _hipcc()
    os.makedirs(BUILD, exist_ok=True)
    objs = []
    cmds = []
    for src in SOURCES:
        obj = os.path.join(BUILD, src.replace(".hip", ".o"))
        objs.append(obj)
        cmds.append([hipcc, *CFLAGS, "-c", os.path.join(CSRC, src), "-o", obj])
    jobs = jobs or min(len(cmds), os.cpu_count() or 4, 8)
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        for out in ex.map(_run, cmds):
            if verbose and out.strip():
                print(out)
    tmp = LIB + ".tmp"
    _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp])
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
