"""Builds libmoe.so (the HIP kernels and the C ABI) for gfx950 with hipcc.

Usage: python -m mxfp4_quantized_weights_amd.build   (or call build()).
Objects go to <repo>/_build/, the shared library next to this file.
"""
from __future__ import annotations

import concurrent.futures
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libmoe.so")
SOURCES = ["api.hip", "route.hip", "quant.hip", "gemm.hip", "diag.hip", "decode.hip"]
ARCH = "gfx950"

# -packed-fp32-ops off: no v_pk_{add,mul,fma}_f32 in the generated code.
# Correctly rounded fp32 division: the quantisers' s = amax/448 and v/s must
# be IEEE divisions to be reproducible.  Denormals are kept (HIP default).
HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++20", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-Wall", "-Wno-unused-function",
]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    return "hipcc"


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if r.returncode != 0:
        raise RuntimeError("build failed:\n" + " ".join(cmd) + "\n" + r.stdout)
    return r.stdout


def build(verbose: bool = False, extra_flags=None) -> str:
    """Compiles every source and links libmoe.so; returns its path."""
    out_dir = os.path.join(ROOT, "_build")
    os.makedirs(out_dir, exist_ok=True)
    hipcc = _hipcc()
    flags = HIPCC_FLAGS + list(extra_flags or [])
    objs = []
    cmds = []
    for src in SOURCES:
        obj = os.path.join(out_dir, src.replace(".hip", ".o"))
        objs.append(obj)
        cmds.append([hipcc, *flags, "-c", os.path.join(CSRC, src), "-o", obj])
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(4, len(cmds))) as ex:
        logs = list(ex.map(_run, cmds))
    tmp = LIB + ".tmp"
    _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp])
    os.replace(tmp, LIB)
    if verbose:
        for cmd, log in zip(cmds, logs):
            print(" ".join(cmd))
            if log.strip():
                print(log)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
