"""The C ABI from C: tests/c_client.c is compiled with gcc as C99 against include/specconv.h
and linked with libspecconv.so, then run (host-side calls only, no GPU needed)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIBDIR = os.path.join(ROOT, "fft_causal_long_amd")


def test_c_client(tmp_path):
    gcc = shutil.which("gcc")
    if gcc is None or not os.path.exists(os.path.join(LIBDIR, "libspecconv.so")):
        pytest.skip("gcc or the built library is missing")
    exe = str(tmp_path / "c_client")
    # the HIP headers expect the platform macro when the compiler is not hipcc
    cmd = [gcc, "-std=c99", "-Wall", "-Werror", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROOT, "include"), "-I", "/opt/rocm/include",
           os.path.join(ROOT, "tests", "c_client.c"), "-L", LIBDIR, "-lspecconv",
           "-Wl,-rpath," + LIBDIR, "-o", exe]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr
    run = subprocess.run([exe], capture_output=True, text=True, timeout=60)
    assert run.returncode == 0, run.stdout + run.stderr
    assert "c client ok" in run.stdout
