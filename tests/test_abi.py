"""The C ABI without a GPU: the library loads, exports every symbol include/specconv.h
declares, and rejects bad arguments on the host before any HIP call (CPU only; no call
here reaches a kernel launch)."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "specconv.h")
LIB = os.path.join(ROOT, "fft_causal_long_amd", "libspecconv.so")


@pytest.fixture(scope="module")
def sc():
    if not os.path.exists(LIB):
        from fft_causal_long_amd import build as b  # noqa: F401  (package import needs the .so)
    import importlib.util
    if not os.path.exists(LIB):
        spec = importlib.util.spec_from_file_location(
            "sc_build", os.path.join(ROOT, "fft_causal_long_amd", "build.py"))
        mod = importlib.util.module_from_spec(spec)
        spec.loader.exec_module(mod)
        mod.build()
    import fft_causal_long_amd as m
    return m


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sc_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for n in ("sc_causal_conv_f32", "sc_causal_conv_bf16", "sc_causal_conv_ntt_i32",
              "sc_workspace_bytes", "sc_causal_conv_ex", "sc_status_string", "sc_version",
              "sc_ntt_range_ok"):
        assert n in names


def test_every_declared_symbol_is_exported(sc):
    h = sc.lib()
    for n in declared_functions():
        assert hasattr(h, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", LIB], capture_output=True, text=True).stdout
    exported = set(re.findall(r" T (sc_\w+)", out))
    assert set(declared_functions()) <= exported
    # nothing but the C ABI leaks out under the sc_ prefix
    assert exported <= set(declared_functions())


def test_links_hip_runtime_by_soname():
    out = subprocess.run(["readelf", "-d", LIB], capture_output=True, text=True).stdout
    assert "libamdhip64.so.7" in out


A, B_, C_ = 0x100000, 0x200000, 0x300000   # fake, never dereferenced


@pytest.mark.parametrize("fn", ["sc_causal_conv_f32", "sc_causal_conv_bf16", "sc_causal_conv_ntt_i32"])
def test_host_validation(sc, fn):
    f = getattr(sc.lib(), fn)
    INVALID, OK = sc.SC_ERR_INVALID_ARGUMENT, sc.SC_OK
    assert f(A, B_, C_, -1, 1, 1, None) == INVALID
    assert f(A, B_, C_, 1, -1, 1, None) == INVALID
    assert f(A, B_, C_, 1, 1, -5, None) == INVALID
    assert f(None, B_, C_, 1, 1, 4, None) == INVALID
    assert f(A, None, C_, 1, 1, 4, None) == INVALID
    assert f(A, B_, None, 1, 1, 4, None) == INVALID
    assert f(A + 1, B_, C_, 1, 1, 4, None) == INVALID          # misaligned
    assert f(A, B_, A, 1, 1, 4, None) == INVALID               # r aliases v
    assert f(A, B_, B_ + 4, 1, 1, 4, None) == INVALID           # r overlaps g
    assert f(A, B_, C_, 2**40, 2**40, 2**40, None) == INVALID  # size overflow
    # empty problems are a successful no-op, even with null pointers
    assert f(None, None, None, 0, 7, 9, None) == OK
    assert f(None, None, None, 3, 7, 0, None) == OK


def test_unsupported_lengths_rejected_before_launch(sc):
    h = sc.lib()
    UNSUP = sc.SC_ERR_UNSUPPORTED
    assert h.sc_causal_conv_ntt_i32(A, B_, C_, 1, 1, 65537, None) == UNSUP   # four-step NTT max
    far = (1 << 32, 2 << 32, 3 << 32)                  # fake, far enough apart not to overlap
    assert h.sc_causal_conv_f32(*far, 1, 1, 2**22 + 1, None) == UNSUP
    opt = sc.sc_options(sc.PATH_FOUR_STEP, -1)         # the split needs L > 2048
    assert h.sc_causal_conv_ex(0, A, B_, C_, 1, 1, 2048, ctypes.byref(opt), None, 0, None) == UNSUP
    opt = sc.sc_options(sc.PATH_FUSED, -1)             # one workgroup holds at most L = 4096
    assert h.sc_causal_conv_ex(0, A, B_, C_, 1, 1, 4097, ctypes.byref(opt), None, 0, None) == UNSUP
    assert h.sc_causal_conv_ex(2, A, B_, C_, 1, 1, 4097, ctypes.byref(opt), None, 0, None) == UNSUP
    # the matrix-core first pass: the M = 4096 kernel with bf16 storage only
    opt = sc.sc_options(sc.PATH_FUSED_MFMA, -1)
    for kind, L in ((0, 4096), (2, 4096), (3, 4096), (1, 2048), (1, 4097), (1, 64)):
        assert h.sc_causal_conv_ex(kind, A, B_, C_, 1, 1, L, ctypes.byref(opt), None, 0,
                                   None) == UNSUP
    # the exact four-step split has rows of 4096: forced only above the fused range
    opt = sc.sc_options(sc.PATH_FOUR_STEP, -1)
    for kind in (2, 3):
        for L in (4096, 65537):
            assert h.sc_causal_conv_ex(kind, A, B_, C_, 1, 1, L, ctypes.byref(opt), None, 0,
                                       None) == UNSUP


def test_options_validation(sc):
    h = sc.lib()
    INVALID = sc.SC_ERR_INVALID_ARGUMENT
    opt = sc.sc_options(0, -1)
    opt.reserved[2] = 1
    assert h.sc_causal_conv_ex(0, A, B_, C_, 1, 1, 64, ctypes.byref(opt), None, 0, None) == INVALID
    opt = sc.sc_options(0, 65)
    assert h.sc_causal_conv_ex(0, A, B_, C_, 1, 1, 64, ctypes.byref(opt), None, 0, None) == INVALID
    opt = sc.sc_options(9, -1)
    assert h.sc_causal_conv_ex(0, A, B_, C_, 1, 1, 64, ctypes.byref(opt), None, 0, None) == INVALID
    opt = sc.sc_options(sc.PATH_DIRECT, -1)    # direct summation is float only
    assert h.sc_causal_conv_ex(2, A, B_, C_, 1, 1, 64, ctypes.byref(opt), None, 0, None) == \
        sc.SC_ERR_UNSUPPORTED
    assert h.sc_causal_conv_ex(7, A, B_, C_, 1, 1, 64, None, None, 0, None) == INVALID


def test_host_helpers(sc):
    assert sc.sc_ntt_range_ok(127, 127, 4096)                  # 66,064,384
    assert sc.sc_ntt_range_ok(1, 499122176, 1)
    assert not sc.sc_ntt_range_ok(1, 499122177, 1)
    assert not sc.sc_ntt_range_ok(2**40, 2**40, 2**40)        # no overflow
    assert not sc.sc_ntt_range_ok(-1, 1, 1)
    assert sc.sc_status_string(0) == "SC_OK"
    assert sc.sc_status_string(4) == "SC_ERR_WORKSPACE"
    assert sc.sc_status_string(99) == "SC_STATUS_UNKNOWN"
    assert sc.sc_version() >= 902
    # sc_prepare: argument checks on the host; an empty length needs no table
    assert sc.sc_prepare(7, 64) == sc.SC_ERR_INVALID_ARGUMENT
    assert sc.sc_prepare(sc.KIND_F32, -1) == sc.SC_ERR_INVALID_ARGUMENT
    assert sc.sc_prepare(sc.KIND_NTT_I32, 65537) == sc.SC_ERR_UNSUPPORTED
    assert sc.sc_prepare(sc.KIND_FIXED_F32, 65537) == sc.SC_ERR_UNSUPPORTED
    assert sc.sc_prepare(sc.KIND_F32, 2**22 + 1) == sc.SC_ERR_UNSUPPORTED
    assert sc.sc_prepare(sc.KIND_BF16, 0) == sc.SC_OK
    assert sc.sc_workspace_bytes(sc.KIND_F32, 8, 1024, 4096) == 0
    # four-step lengths need scratch; the exact path and bad shapes need none
    assert sc.sc_workspace_bytes(sc.KIND_F32, 1, 1536, 65536) > 0
    assert sc.sc_workspace_bytes(sc.KIND_BF16, 1, 1, 5000) > 0
    assert sc.sc_workspace_bytes(sc.KIND_NTT_I32, 1, 1, 4096) == 0
    # the exact four-step path: 24 M bytes per channel (T: 2 branches x 2 arrays, S: 2 branches
    # of M int32), chunked
    assert sc.sc_workspace_bytes(sc.KIND_NTT_I32, 1, 3, 5000) == 3 * 24 * 8192
    assert sc.sc_workspace_bytes(sc.KIND_NTT_I32, 1, 1, 65536) == 24 * 65536
    assert sc.sc_workspace_bytes(sc.KIND_NTT_I32, 1, 1, 65537) == 0
    assert sc.sc_workspace_bytes(sc.KIND_F32, -1, 1, 65536) == 0
    assert sc.sc_workspace_bytes(sc.KIND_F32, 1, 1, 2**23) == 0      # above the maximum


D_, E_ = 0x400000, 0x500000   # fake output pointers of the gradient calls


def test_header_declares_the_gradient_calls():
    names = declared_functions()
    for n in ("sc_causal_conv_bwd_f32", "sc_causal_conv_bwd_bf16", "sc_causal_conv_bwd_ntt_i32",
              "sc_causal_conv_bwd_ex"):
        assert n in names


@pytest.mark.parametrize("fn", ["sc_causal_conv_bwd_f32", "sc_causal_conv_bwd_bf16",
                                "sc_causal_conv_bwd_ntt_i32"])
def test_bwd_host_validation(sc, fn):
    f = getattr(sc.lib(), fn)
    INVALID, OK = sc.SC_ERR_INVALID_ARGUMENT, sc.SC_OK
    good = [A, B_, C_, D_, E_]
    assert f(*good, -1, 1, 1, None) == INVALID
    assert f(*good, 1, 1, -2, None) == INVALID
    for i in range(5):                                   # each pointer null
        p = list(good)
        p[i] = None
        assert f(*p, 1, 1, 4, None) == INVALID, i
    for i in range(5):                                   # each pointer misaligned
        p = list(good)
        p[i] += 1
        assert f(*p, 1, 1, 4, None) == INVALID, i
    for out in (3, 4):                                   # an output on any input or the other output
        for other in range(5):
            if other == out:
                continue
            p = list(good)
            p[out] = p[other] + 4
            assert f(*p, 1, 1, 4, None) == INVALID, (out, other)
    assert f(*good, 2**40, 2**40, 2**40, None) == INVALID
    assert f(None, None, None, None, None, 0, 5, 5, None) == OK
    assert f(None, None, None, None, None, 5, 5, 0, None) == OK


def test_bwd_unsupported_and_options(sc):
    h = sc.lib()
    UNSUP, INVALID = sc.SC_ERR_UNSUPPORTED, sc.SC_ERR_INVALID_ARGUMENT
    assert h.sc_causal_conv_bwd_ntt_i32(A, B_, C_, D_, E_, 1, 1, 65537, None) == UNSUP
    far = [k << 32 for k in range(1, 6)]
    assert h.sc_causal_conv_bwd_f32(*far, 1, 1, 2**22 + 1, None) == UNSUP
    opt = sc.sc_options(sc.PATH_FUSED, -1)
    assert h.sc_causal_conv_bwd_ex(0, A, B_, C_, D_, E_, 1, 1, 4097, ctypes.byref(opt), None, 0,
                                   None) == UNSUP
    opt = sc.sc_options(0, -1)
    opt.reserved[0] = 3
    assert h.sc_causal_conv_bwd_ex(1, A, B_, C_, D_, E_, 1, 1, 64, ctypes.byref(opt), None, 0,
                                   None) == INVALID
    assert h.sc_causal_conv_bwd_ex(5, A, B_, C_, D_, E_, 1, 1, 64, None, None, 0, None) == INVALID
    assert sc.sc_version() >= 200


def test_fixed_kind_host_checks(sc):
    h = sc.lib()
    INVALID, UNSUP = sc.SC_ERR_INVALID_ARGUMENT, sc.SC_ERR_UNSUPPORTED
    f = h.sc_causal_conv_fixed_f32
    assert f(A, B_, C_, 1, 1, 64, 65, 0, None) == INVALID            # fraction bits in [-64, 64]
    assert f(A, B_, C_, 1, 1, 64, 0, -65, None) == INVALID
    assert f(A, B_, C_, 1, 1, 65537, 20, 20, None) == UNSUP           # exact paths: L <= 65536
    assert f(A, B_, A, 1, 1, 64, 20, 20, None) == INVALID             # r aliases v
    assert f(None, None, None, 0, 1, 64, 20, 20, None) == sc.SC_OK
    # fraction bits are only meaningful for the fixed kind
    opt = sc.sc_options(0, -1, 3, 0)
    assert h.sc_causal_conv_ex(0, A, B_, C_, 1, 1, 64, ctypes.byref(opt), None, 0, None) == INVALID
    # no gradients for the fixed kind
    assert h.sc_causal_conv_bwd_ex(3, A, B_, C_, D_, E_, 1, 1, 64, None, None, 0, None) == UNSUP
    # up to L = 4096 one kernel keeps the three residues of an output in registers: no
    # scratch; beyond, the four-step split per prime: 40 M bytes per channel (M = 2^ceil(lg L))
    assert sc.sc_workspace_bytes(sc.KIND_FIXED_F32, 2, 3, 100) == 0
    assert sc.sc_workspace_bytes(sc.KIND_FIXED_F32, 8, 1024, 4096) == 0
    assert sc.sc_workspace_bytes(sc.KIND_FIXED_F32, 1, 1, 5000) == 40 * 8192
    assert sc.sc_workspace_bytes(sc.KIND_FIXED_F32, 2, 3, 65536) == 6 * 40 * 65536
    assert sc.sc_workspace_bytes(sc.KIND_FIXED_F32, 1, 1, 65537) == 0
    assert sc.sc_blc_workspace_bytes(sc.KIND_FIXED_F32, 2, 100, 3) == \
        3 * (((2 * 3 * 100 * 4) + 255) // 256 * 256)


def test_fixed_range_helper(sc):
    ok = sc.sc_fixed_range_ok
    assert ok(8.0, 1.0, 24, 24, 4096)             # 4096 * 2^27 * 2^24 = 2^63
    assert not ok(8.0, 1.0, 40, 40, 4096)         # 2^12 * 2^43 * 2^40 > 2^87.6
    assert not ok(1.0, 1.0, 51, 0, 1)             # an encoding reaches 2^51
    assert ok(1.0, 1.0, 50, 0, 1)
    assert not ok(float("nan"), 1.0, 0, 0, 1)
    assert not ok(1.0, 1.0, 65, 0, 1)
    assert ok(0.0, 0.0, 64, 64, 4096)
    # the boundary: L * 2^43 * 2^43 against (P - 1) / 2 with P ~ 2^88.6
    P = 998244353 * 1004535809 * 469762049
    L = ((P - 1) // 2) // (2 ** 86)
    assert ok(2.0 ** 43, 2.0 ** 43, 0, 0, L)
    assert not ok(2.0 ** 43, 2.0 ** 43, 0, 0, L + 1)


def test_shared_filter_host_checks(sc):
    h = sc.lib()
    INVALID, UNSUP, OK = sc.SC_ERR_INVALID_ARGUMENT, sc.SC_ERR_UNSUPPORTED, sc.SC_OK
    # spectrum size: C * (2M + 32) float2, M = max(64, next_pow2(L)); 0 for unsupported L
    assert sc.sc_filter_spectrum_bytes(3, 100) == 3 * (2 * 128 + 32) * 8
    assert sc.sc_filter_spectrum_bytes(1, 1) == (2 * 64 + 32) * 8
    assert sc.sc_filter_spectrum_bytes(1, 4097) == 0
    assert sc.sc_filter_spectrum_bytes(-1, 64) == 0
    for name in ("sc_filter_spectrum_f32", "sc_filter_spectrum_bf16"):
        f = getattr(h, name)
        assert f(A, B_, 4, 5000, None) == UNSUP
        assert f(None, B_, 4, 64, None) == INVALID
        assert f(A, None, 4, 64, None) == INVALID
        assert f(A, B_ + 4, 4, 64, None) == INVALID            # spectrum not 8-byte aligned
        assert f(A, A + 64, 4, 64, None) == INVALID            # spectrum overlaps k
        assert f(A, B_, -1, 64, None) == INVALID
        assert f(None, None, 0, 64, None) == OK
    for name in ("sc_causal_conv_spec_f32", "sc_causal_conv_spec_bf16",
                 "sc_causal_conv_shared_f32", "sc_causal_conv_shared_bf16"):
        f = getattr(h, name)
        assert f(A, B_, C_, 2, 4, 5000, None) == UNSUP, name
        assert f(None, B_, C_, 2, 4, 64, None) == INVALID, name
        assert f(A, None, C_, 2, 4, 64, None) == INVALID, name
        assert f(A, B_, None, 2, 4, 64, None) == INVALID, name
        assert f(A, B_, A + 8, 2, 4, 64, None) == INVALID, name   # r overlaps v
        assert f(A, B_, B_, 2, 4, 64, None) == INVALID, name      # r overlaps k / spectrum
        assert f(A, B_, C_, -2, 4, 64, None) == INVALID, name
        assert f(None, None, None, 0, 4, 64, None) == OK, name
    # one filter set must fit a 32-bit span: C * L * 4 bytes < 2^31
    assert h.sc_causal_conv_shared_f32(1 << 40, 2 << 40, 3 << 40, 1, 1 << 19, 4096, None) == UNSUP


def test_shared_filter_bwd_host_checks(sc):
    h = sc.lib()
    INVALID, UNSUP, OK = sc.SC_ERR_INVALID_ARGUMENT, sc.SC_ERR_UNSUPPORTED, sc.SC_OK
    for name in ("sc_causal_conv_spec_bwd_f32", "sc_causal_conv_spec_bwd_bf16",
                 "sc_causal_conv_shared_bwd_f32", "sc_causal_conv_shared_bwd_bf16"):
        f = getattr(h, name)
        assert f(A, B_, C_, D_, E_, 2, 4, 5000, None) == UNSUP, name
        for i in range(5):                                        # any null pointer
            args = [A, B_, C_, D_, E_]
            args[i] = None
            assert f(*args, 2, 4, 64, None) == INVALID, (name, i)
        assert f(A, B_, C_, A + 8, E_, 2, 4, 64, None) == INVALID, name   # dv overlaps dr
        assert f(A, B_, C_, D_, B_ + 8, 2, 4, 64, None) == INVALID, name  # dk overlaps v
        assert f(A, B_, C_, D_, C_, 2, 4, 64, None) == INVALID, name      # dk overlaps k
        assert f(A, B_, C_, D_, D_ + 64, 2, 4, 64, None) == INVALID, name  # dk overlaps dv
        assert f(A, B_, C_, D_ + 1, E_, 2, 4, 64, None) == INVALID, name  # misaligned dv
        assert f(A, B_, C_, D_, E_, -2, 4, 64, None) == INVALID, name
        # no rows: nothing to read, but dk (C x L) is written (zero), so it must be given
        assert f(None, None, None, None, None, 4, 0, 64, None) == OK, name
        assert f(None, None, None, None, None, 0, 4, 0, None) == OK, name
        assert f(None, None, None, None, None, 0, 4, 64, None) == INVALID, name
        assert f(None, None, None, None, E_ + 1, 0, 4, 64, None) == INVALID, name
    assert h.sc_causal_conv_spec_bwd_f32(A, B_, C_ + 4, D_, E_, 2, 4, 64, None) == INVALID
    # the row loops count batch rows in 32 bits: B = 2^31 (4 GB of bf16 at C = L = 1) is
    # refused before any HIP call instead of being truncated
    big = [k << 40 for k in range(1, 6)]
    for name in ("sc_causal_conv_spec_bwd_bf16", "sc_causal_conv_shared_bwd_bf16"):
        assert getattr(h, name)(*big, 1 << 31, 1, 1, None) == UNSUP, name
    assert h.sc_causal_conv_shared_bwd_f32(1 << 40, 2 << 40, 3 << 40, 4 << 40, 5 << 40, 1,
                                           1 << 19, 4096, None) == UNSUP


def test_token_major_host_checks(sc):
    h = sc.lib()
    INVALID, UNSUP, OK, WS = (sc.SC_ERR_INVALID_ARGUMENT, sc.SC_ERR_UNSUPPORTED, sc.SC_OK,
                              sc.SC_ERR_WORKSPACE)
    F32, BF16, NTT = sc.KIND_F32, sc.KIND_BF16, sc.KIND_NTT_I32
    MiB = 1 << 20
    # whole batch rows per chunk while a row fits one third of the 96 MiB staging budget:
    # here 2 rows of 4M float32 or 4 rows of 4M bfloat16
    assert sc.sc_blc_workspace_bytes(F32, 8, 4096, 1024) == 3 * 32 * MiB
    assert sc.sc_blc_workspace_bytes(BF16, 8, 4096, 1024) == 3 * 32 * MiB
    assert sc.sc_blc_workspace_bytes(F32, 1, 256, 64) == 3 * 64 * 1024
    # longer rows: blocks of 64k channels, plus the four-step scratch of one block
    inner = sc.sc_workspace_bytes(F32, 1, 128, 65536)
    assert inner > 0
    assert sc.sc_blc_workspace_bytes(F32, 1, 65536, 1536) == 3 * 32 * MiB + (inner + 255) // 256 * 256
    # the exact kind above 4096: three staging buffers plus the four-step NTT's 24 M bytes
    # per channel
    assert sc.sc_blc_workspace_bytes(NTT, 1, 8192, 4) == 3 * 4 * 8192 * 4 + 4 * 24 * 8192
    assert sc.sc_blc_workspace_bytes(NTT, 1, 65537, 4) == 0         # beyond the exact paths
    assert sc.sc_blc_workspace_bytes(F32, 0, 64, 4) == 0
    assert sc.sc_blc_workspace_bytes(7, 1, 64, 4) == 0

    opt = sc.sc_options(0, -1)
    W = 0x10000000           # a fake 256-aligned workspace far from A, B_, C_
    need = sc.sc_blc_workspace_bytes(F32, 2, 64, 4)
    f = h.sc_causal_conv_blc_ex
    assert f(F32, A, B_, C_, 2, 64, 4, None, W, need - 1, None) == WS
    assert f(F32, A, B_, C_, 2, 64, 4, None, W + 8, need, None) == INVALID     # alignment
    assert f(F32, A, B_, C_, 2, 64, 4, None, A - 256, need, None) == INVALID  # ws overlaps v
    assert f(F32, A, B_, C_, 2, 64, 4, None, None, 16, None) == INVALID       # bytes, no ws
    assert f(F32, None, B_, C_, 2, 64, 4, None, W, need, None) == INVALID
    assert f(F32, A, B_, A + 4, 2, 64, 4, None, W, need, None) == INVALID     # r overlaps v
    assert f(F32, A, B_, C_, -1, 64, 4, None, W, need, None) == INVALID
    assert f(F32, A, B_, C_, 2, 64, 4, ctypes.byref(sc.sc_options(9, -1)), W, need,
             None) == INVALID
    assert f(NTT, A, B_, C_, 1, 65537, 1, None, None, 0, None) == UNSUP     # beyond the exact paths
    assert f(F32, 1 << 40, 2 << 40, 3 << 40, 1, (1 << 22) + 1, 1, None, None, 0, None) == UNSUP
    assert f(F32, None, None, None, 0, 64, 4, ctypes.byref(opt), None, 0, None) == OK
    for name in ("sc_causal_conv_blc_f32", "sc_causal_conv_blc_bf16"):
        g = getattr(h, name)
        assert g(None, B_, C_, 2, 64, 4, None) == INVALID, name
        assert g(A, B_, B_ + 2, 2, 64, 4, None) == INVALID, name
        assert g(None, None, None, 2, 0, 4, None) == OK, name


def test_gate_host_checks(sc):
    h = sc.lib()
    INVALID, UNSUP, OK, WS = (sc.SC_ERR_INVALID_ARGUMENT, sc.SC_ERR_UNSUPPORTED, sc.SC_OK,
                              sc.SC_ERR_WORKSPACE)
    F32, BF16, NTT = sc.KIND_F32, sc.KIND_BF16, sc.KIND_NTT_I32
    MiB = 1 << 20
    for name in ("sc_gate_f32", "sc_gate_bf16"):
        f = getattr(h, name)
        assert f(A, B_, C_, 1, 100, 16, None) == UNSUP, name           # C not a multiple of 64
        assert f(None, B_, C_, 1, 64, 16, None) == INVALID, name
        assert f(A, None, C_, 1, 64, 16, None) == INVALID, name
        assert f(A, B_, None, 1, 64, 16, None) == INVALID, name
        assert f(A, B_, A + 64, 1, 64, 16, None) == INVALID, name       # g overlaps s
        assert f(A, B_, B_ + 64, 1, 64, 16, None) == INVALID, name      # g overlaps W
        assert f(A + 1, B_, C_, 1, 64, 16, None) == INVALID, name       # misaligned
        assert f(A, B_ + 4, C_, 1, 64, 16, None) == INVALID, name       # W not 16-byte aligned
        assert f(A, B_, C_, -1, 64, 16, None) == INVALID, name
        assert f(None, None, None, 0, 64, 16, None) == OK, name
    # staging: one g buffer (channel-major, the whole budget) or v, g, r buffers (token-major)
    assert sc.sc_gate_conv_workspace_bytes(BF16, 8, 1024, 4096) == 64 * MiB
    assert sc.sc_gate_conv_blc_workspace_bytes(BF16, 8, 4096, 1024) == 3 * 32 * MiB
    assert sc.sc_gate_conv_workspace_bytes(F32, 1, 100, 64) == 0     # C not a multiple of 64
    assert sc.sc_gate_conv_workspace_bytes(NTT, 1, 64, 64) == 0
    D, E = 0x400000, 0x500000
    W = 0x10000000
    for name in ("sc_gate_conv_ex", "sc_gate_conv_blc_ex"):
        f = getattr(h, name)
        # argument order (v, s, W, r) and sizes B, then C, L (channel-major) or L, C
        sizes = (1, 64, 16) if name == "sc_gate_conv_ex" else (1, 16, 64)
        need = (sc.sc_gate_conv_workspace_bytes(F32, 1, 64, 16) if name == "sc_gate_conv_ex"
                else sc.sc_gate_conv_blc_workspace_bytes(F32, 1, 16, 64))
        assert need > 0
        assert f(NTT, A, B_, C_, D, *sizes, None, None, 0, None) == INVALID, name
        assert f(F32, A, B_, None, D, *sizes, None, None, 0, None) == INVALID, name
        assert f(F32, A, B_, C_, A + 4, *sizes, None, None, 0, None) == INVALID, name  # r on v
        assert f(F32, A, B_, C_, C_ + 4, *sizes, None, None, 0, None) == INVALID, name  # r on W
        assert f(F32, A, B_, C_, D, *sizes, None, W, need - 1, None) == WS, name
        assert f(F32, A, B_, C_, D, *sizes, None, W + 8, need, None) == INVALID, name
        assert f(F32, None, None, None, None, 0, *sizes[1:], None, None, 0, None) == OK, name
    bad = (1, 100, 16)
    assert h.sc_gate_conv_ex(F32, A, B_, C_, D, *bad, None, None, 0, None) == UNSUP
    # token-major s must be 16-byte aligned (row vectors)
    assert h.sc_gate_conv_blc_ex(F32, A, B_ + 4, C_, D, 1, 16, 64, None, None, 0, None) == INVALID


def test_tensor_front_end_refuses_host_tensors(sc):
    # there is no CPU path: host tensors are refused before any library call
    import torch
    v = torch.ones(1, 2, 8)
    calls = [lambda: sc.causal_conv(v, v), lambda: sc.causal_conv_blc(v, v),
             lambda: sc.causal_conv_bwd(v, v, v), lambda: sc.causal_conv_fixed(v, v, 8, 8),
             lambda: sc.filter_spectrum(v[0]), lambda: sc.gate(torch.ones(1, 64, 8), torch.ones(64, 64, 3))]
    for call in calls:
        with pytest.raises(ValueError, match="GPU"):
            call()


def test_package_without_its_library_fails_to_import(tmp_path):
    # the Python package with no libspecconv.so beside it raises on import (no fallback)
    import shutil
    pkg = tmp_path / "fft_causal_long_amd"
    pkg.mkdir()
    for name in ("__init__.py", "build.py"):
        shutil.copy(os.path.join(ROOT, "fft_causal_long_amd", name), pkg / name)
    p = subprocess.run(["python", "-c", "import fft_causal_long_amd"], cwd=str(tmp_path),
                       env=dict(os.environ, PYTHONPATH=str(tmp_path)), capture_output=True,
                       text=True, timeout=120)
    assert p.returncode != 0
    assert "libspecconv.so is not built" in p.stderr
