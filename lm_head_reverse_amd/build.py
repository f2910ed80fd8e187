"""Build librkl.so (HIP, gfx950) in-tree with hipcc.

    python -m lm_head_reverse_amd.build          # writes lm_head_reverse_amd/librkl.so
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
LIB = os.path.join(PKG, "librkl.so")
SOURCES = ["rkl_kernels.hip", "rkl_api.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for c in (os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc"), shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build librkl.so)")


def build(verbose: bool = False, extra: list[str] | None = None) -> str:
    """Compile every source for gfx950 and link librkl.so; returns its path."""
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared", "-fvisibility=hidden",
           # packed-fp32 instructions are kept out of the generated code
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-Wall", "-Wno-unused-function",
           f"-I{INCLUDE}", f"-I{CSRC}",
           *[os.path.join(CSRC, s) for s in SOURCES],
           "-o", tmp]
    if extra:
        cmd[1:1] = extra
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError(f"hipcc failed ({r.returncode})")
    noise = "'-packed-fp32-ops' is not a recognized feature"
    msgs = [l for l in (r.stdout + r.stderr).splitlines() if l.strip() and noise not in l]
    if msgs and verbose:
        print("\n".join(msgs))
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
