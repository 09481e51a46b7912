"""Build the C-ABI library ``liblora_sgmv.so`` in-tree with hipcc for gfx950.

    python -m segmented_gather_matmul_amd.build
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "liblora_sgmv.so")
SOURCES = [os.path.join(CSRC, "lora_kernels.hip"), os.path.join(CSRC, "lora_pool.hip"),
           os.path.join(CSRC, "lora_host.cpp")]
HEADERS = [os.path.join(INCLUDE, "lora_sgmv.h"), os.path.join(CSRC, "lora_internal.hpp")]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def flags() -> list[str]:
    return ["-O3", "-std=c++17", "-fPIC", "-shared", f"--offload-arch={ARCH}",
            # Packed FP32 instructions stay off: plain float code is compiled to scalar FP32 ops.
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            # Leading scalar kernel arguments (up to four; only the hand-off kernel has any
            # before its argument block) arrive preloaded in scalar registers.
            "-mllvm", "-amdgpu-kernarg-preload-count=4",
            "-Wall", "-Wno-unused-function", f"-I{INCLUDE}", f"-I{CSRC}"]


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp"
    cmd = [hipcc(), *flags(), *SOURCES, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed building liblora_sgmv.so")
    os.replace(tmp, LIB)
    return LIB


def stale() -> bool:
    if not os.path.exists(LIB):
        return True
    t = os.path.getmtime(LIB)
    return any(os.path.getmtime(p) > t for p in SOURCES + HEADERS)


if __name__ == "__main__":
    print(build(verbose=True))
