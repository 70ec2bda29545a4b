"""The build script's commands (no compiler run): every source is compiled for gfx950 with
packed fp32 instructions disabled, and only the files measured to gain from it take the
memory-clause instruction schedule."""
import importlib.util
import os

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _build_module():
    spec = importlib.util.spec_from_file_location(
        "_sc_build_cmds", os.path.join(ROOT, "fft_causal_long_amd", "build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_every_source_has_the_common_options():
    b = _build_module()
    srcs = b.sources()
    assert any(s.endswith("sc_fused4k.hip") for s in srcs)
    assert any(s.endswith("sc_host.cpp") for s in srcs)
    for s in srcs:
        cmd = b.compile_command(s, "/tmp/x.o")
        assert "--offload-arch=gfx950" in cmd
        i = cmd.index("-packed-fp32-ops")
        assert cmd[i - 1] == "-Xclang" and cmd[i - 2] == "-target-feature"
        assert "-c" in cmd and cmd[-3] == s


def test_schedule_option_only_where_measured():
    b = _build_module()
    flag = "-amdgpu-sched-strategy=max-memory-clause"
    for s in b.sources():
        has = flag in b.compile_command(s, "/tmp/x.o")
        assert has == (os.path.basename(s) in ("sc_fused4k.hip", "sc_ntt.hip")), s


def test_link_produces_one_shared_library():
    b = _build_module()
    cmd = b.link_command(["a.o", "b.o"], "/tmp/lib.so")
    assert "-shared" in cmd and cmd[-2:] == ["-o", "/tmp/lib.so"]
