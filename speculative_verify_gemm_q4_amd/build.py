"""Build the gfx950 library ``libq4verify.so`` in-tree with hipcc.

The library is the product: every step of the verify GEMM runs in its HIP
kernels.  Flags: gfx950 only, -O3, packed-fp32 instructions disabled (the
host pass warns that it does not know that feature; the warning is expected).
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libq4verify.so")
SOURCES = [os.path.join(CSRC, "q4verify_host.cpp"),
           os.path.join(CSRC, "q4verify_kernels.hip"),
           os.path.join(CSRC, "q4verify_sample.hip"),
           os.path.join(CSRC, "q4verify_gdn.hip"),
           os.path.join(CSRC, "q4verify_attn.hip")]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
         "-Wall", "-Wextra", "-Wno-unused-parameter",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         # MFMA results in VGPRs: the epilogue reads them without moves
         "-mllvm", "-amdgpu-mfma-vgpr-form",
         # kernel arguments arrive in SGPRs at wave launch (no scalar load
         # round trip before a kernel's first memory access)
         "-mllvm", "-amdgpu-kernarg-preload-count=16",
         "-I", INCLUDE, "-I", CSRC]


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp"
    cmd = [HIPCC, *FLAGS, "-o", tmp, *SOURCES]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "'-packed-fp32-ops' is not a recognized feature"
    err = "\n".join(line for line in res.stderr.splitlines() if noise not in line)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{err}")
    if err.strip() and verbose:
        print(err, file=sys.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
