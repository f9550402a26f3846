"""Build libwoq.so in-tree with hipcc for gfx950.

    python -m weight_only_quantized_quantize_amd.build

Compiles the host C++ and the HIP device code into one shared library next to
this file.  Always rebuilds (a few tens of seconds).
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libwoq.so")
ARCH = os.environ.get("WOQ_OFFLOAD_ARCH", "gfx950")

HOST_SOURCES = ["woq_host.cpp", "woq_pool.cpp"]
DEVICE_SOURCES = ["woq_device.hip", "woq_runtime.hip", "woq_pager.cpp", "woq_prep.hip", "woq_noalloc.hip"]

COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function", f"-I{INCLUDE}", f"-I{CSRC}"]
# packed-fp32 VALU ops are kept out of the device code
DEVICE_FLAGS = [f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(ln for ln in r.stdout.splitlines() if "packed-fp32-ops" not in ln and "ignoring feature" not in ln)
    if r.returncode != 0:
        raise RuntimeError(f"build failed: {' '.join(cmd)}\n{out}")
    return out


def build(verbose: bool = False) -> str:
    cc = hipcc()
    srcs = [s for s in DEVICE_SOURCES if os.path.exists(os.path.join(CSRC, s))]
    with tempfile.TemporaryDirectory(prefix="woq_build_") as tmp:
        objs = []
        for s in HOST_SOURCES:
            o = os.path.join(tmp, s + ".o")
            _run([cc, "-x", "c++", *COMMON, "-c", os.path.join(CSRC, s), "-o", o])
            objs.append(o)
        for s in srcs:
            o = os.path.join(tmp, s + ".o")
            out = _run([cc, "-x", "hip", *COMMON, *DEVICE_FLAGS, "-c", os.path.join(CSRC, s), "-o", o])
            if verbose and out.strip():
                print(out)
            objs.append(o)
        tmp_lib = LIB + ".tmp"
        _run([cc, "-shared", f"--offload-arch={ARCH}", *objs, "-o", tmp_lib, "-lpthread"])
        os.replace(tmp_lib, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
