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


# Per-source device-code options.  The M = 4096 fused kernel is scheduled to group its
# memory instructions into clauses: measured in alternating processes on one box, with
# bit-identical outputs, the Medium bf16 call took 0.1427-0.1446 ms against 0.1446-0.1455
# (median of five rounds of 50 calls, four repetitions) and the fp32 one 0.1574 against
# 0.1630.  The same schedule for the whole library made the four-step calls 2-5% slower, so
# it applies to the files that gain from it: the M = 4096 kernel's and the fused NTT
# kernel's (the exact workload's call 0.1531-0.1540 against 0.1551-0.1558 ms).  The fused
# exact real-valued kernel, in a file of its own, was 0.7% slower with it.
_CLAUSES = ["-mllvm", "-amdgpu-sched-strategy=max-memory-clause"]
EXTRA = {"sc_fused4k.hip": _CLAUSES, "sc_ntt.hip": _CLAUSES}


def compile_command(src: str, obj: str) -> list[str]:
    return [
        hipcc(), "-O3", "-std=c++17", "-fPIC", "-c",
        "--offload-arch=" + ARCH,
        # keep the compiler from forming packed fp32 instructions
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-Wall", "-Wno-unused-function",
        "-I", INCLUDE, "-I", CSRC,
        *EXTRA.get(os.path.basename(src), []),
        src, "-o", obj,
    ]


def link_command(objs: list[str], out: str) -> list[str]:
    return [hipcc(), "-shared", "-fPIC", "--offload-arch=" + ARCH, *objs, "-o", out]


def _quiet(stderr: str) -> list[str]:
    # the host pass does not know the packed-fp32 feature flag; drop that noise
    return [l for l in stderr.splitlines()
            if l.strip() and "packed-fp32-ops" not in l and not l.startswith("1 warning")]


def build(verbose: bool = False) -> str:
    """Compile each source to an object (in parallel), then link the shared library."""
    import tempfile
    from concurrent.futures import ThreadPoolExecutor

    tmpdir = tempfile.mkdtemp(prefix="specconv_build_")
    try:
        srcs = sources()
        objs = [os.path.join(tmpdir, os.path.basename(s) + ".o") for s in srcs]
        cmds = [compile_command(s, o) for s, o in zip(srcs, objs)]
        if verbose:
            for c in cmds:
                print(" ".join(c), flush=True)
        jobs = max(1, min(len(cmds), os.cpu_count() or 1, 16))
        with ThreadPoolExecutor(jobs) as ex:
            results = list(ex.map(lambda c: subprocess.run(c, capture_output=True, text=True),
                                  cmds))
        for c, res in zip(cmds, results):
            if res.returncode != 0:
                sys.stderr.write(res.stdout + res.stderr)
                raise RuntimeError("hipcc failed on %s" % c[-3])
            lines = _quiet(res.stderr)
            if verbose and lines:
                sys.stderr.write("\n".join(lines) + "\n")
        tmp = LIB + ".tmp%d" % os.getpid()
        cmd = link_command(objs, tmp)
        if verbose:
            print(" ".join(cmd), flush=True)
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            sys.stderr.write(res.stdout + res.stderr)
            raise RuntimeError("linking libspecconv.so failed")
        os.replace(tmp, LIB)
    finally:
        shutil.rmtree(tmpdir, ignore_errors=True)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
