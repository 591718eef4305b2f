"""Build libaatc.so (host calibration + gfx950 HIP kernels) in-tree with hipcc.

    python -m quantized_attention_klt_amd.build
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIBDIR = os.path.join(PKG, "lib")
LIB = os.path.join(LIBDIR, "libaatc.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
          "-I" + os.path.join(ROOT, "include")]
# Packed FP32 instructions are kept out of the device code.
DEVICE_FLAGS = ["--offload-arch=" + ARCH, "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                "-munsafe-fp-atomics"]


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith((".cpp", ".hip")))


def build(verbose: bool = False) -> str:
    os.makedirs(LIBDIR, exist_ok=True)
    objs = []
    for src in sources():
        obj = os.path.join(LIBDIR, os.path.basename(src) + ".o")
        if src.endswith(".hip"):
            cmd = [HIPCC, "-x", "hip", *COMMON, *DEVICE_FLAGS, "-c", src, "-o", obj]
        else:
            cmd = [HIPCC, "-x", "c++", *COMMON, "-c", src, "-o", obj]
        run(cmd, verbose)
        objs.append(obj)
    tmp = LIB + ".tmp"
    run([HIPCC, "-shared", "--offload-arch=" + ARCH, "-o", tmp, *objs, "-lpthread"], verbose)
    os.replace(tmp, LIB)
    for o in objs:
        os.remove(o)
    return LIB


def run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                    if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError("build failed:\n" + " ".join(cmd) + "\n" + out)
    if verbose and out.strip():
        print(out)


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
