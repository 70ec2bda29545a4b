"""Build libspecconv.so in-tree with hipcc for gfx950.

    python -m fft_causal_long_amd.build          # or: python fft_causal_long_amd/build.py

The library is built from csrc/*.hip and csrc/*.cpp with the public header in include/.
It links the HIP runtime by soname (libamdhip64.so.7), so a process that has already
loaded PyTorch's copy of the runtime keeps using that one copy.
"""
from __future__ import annotations

import glob
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libspecconv.so")
ARCH = os.environ.get("SPECCONV_ARCH", "gfx950")


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (set HIPCC)")


def sources() -> list[str]:
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.cpp")))


def command(out: str) -> list[str]:
    return [
        hipcc(), "-O3", "-std=c++17", "-fPIC", "-shared",
        "--offload-arch=" + ARCH,
        # keep the compiler from forming packed fp32 instructions
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-Wall", "-Wno-unused-function",
        "-I", INCLUDE, "-I", CSRC,
        *sources(), "-o", out,
    ]


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = command(tmp)
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed building libspecconv.so")
    if verbose and res.stderr.strip():
        # the host pass does not know the packed-fp32 feature flag; drop that noise
        lines = [l for l in res.stderr.splitlines() if "packed-fp32-ops" not in l]
        if lines:
            sys.stderr.write("\n".join(lines) + "\n")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
