"""GPU parity of the token-major calls (sc_causal_conv_blc_*): v, g, r in (B, L, C).

The result is checked against the oracle (the float64 direct sum, or the exact int64 sum for
the NTT kind) on the channel-major view of the same stored inputs, to the same bounds as the
channel-major calls, and bit for bit against the channel-major call on the transposed
inputs: both run the same kernels on the same channel data.
"""
import numpy as np
import pytest
import torch

import oracle
from tests.gpu_util import assert_within_bound, to_device, to_host
from workloads import WORKLOADS, make_inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def sc():
    import fft_causal_long_amd as m
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return m


def token_major(x):
    """(B, C, L) -> (B, L, C), contiguous."""
    return np.ascontiguousarray(np.swapaxes(x, 1, 2))


def blc_and_reference(sc, v, g, **kw):
    """r of the token-major call, in (B, C, L), and the channel-major call's r."""
    r_tm = to_host(sc.causal_conv_blc(to_device(token_major(v)), to_device(token_major(g)), **kw))
    r_cm = to_host(sc.causal_conv(to_device(v), to_device(g), **kw))
    r = np.ascontiguousarray(np.swapaxes(r_tm, 1, 2))
    assert np.array_equal(r.view(np.uint8), r_cm.view(np.uint8)), "token-major != channel-major"
    return r


@pytest.mark.parametrize("L", [1, 2, 33, 100, 1024, 3000, 4096])
@pytest.mark.parametrize("C", [5, 64, 130])
def test_f32_against_oracle(sc, L, C):
    v, g = make_inputs(WORKLOADS[2], B=2, C=C, L=L, seed_offset=L * 7 + C)
    print("case blc f32 L=%d C=%d" % (L, C), flush=True)
    r = blc_and_reference(sc, v, g)
    ref, S = oracle.causal_conv_f64(v, g)
    assert_within_bound(r, ref, S, False, "blc f32 L=%d C=%d" % (L, C))


@pytest.mark.parametrize("B,L,C", [(3, 4096, 64), (1, 1000, 100)])
def test_bf16_against_oracle(sc, B, L, C):
    v, g = make_inputs(WORKLOADS[3], B=B, C=C, L=L, seed_offset=B + L + C)
    print("case blc bf16 B=%d L=%d C=%d" % (B, L, C), flush=True)
    r = blc_and_reference(sc, v, g)
    ref, S = oracle.causal_conv_f64(v, g)
    assert_within_bound(r, ref, S, True, "blc bf16 B=%d L=%d C=%d" % (B, L, C))


@pytest.mark.parametrize("L", [1, 77, 4096])
def test_ntt_bit_exact(sc, L):
    v, g = make_inputs(WORKLOADS[5], B=2, C=70, L=L, seed_offset=L)
    print("case blc ntt L=%d" % L, flush=True)
    r = blc_and_reference(sc, v, g)
    ref = oracle.lift_mod_p(oracle.causal_conv_i64(v, g))
    assert np.array_equal(r, ref.astype(np.int32))


def test_channel_blocks_and_four_step(sc):
    # C L above 2^23 elements: one batch row per chunk, channels in blocks of 1024 with a
    # ragged last block of 76; L = 8192 runs on the four-step path
    B, L, C = 2, 8192, 1100
    v, g = make_inputs(WORKLOADS[4], B=B, C=C, L=L, seed_offset=3)
    print("case blc channel blocks B=%d L=%d C=%d" % (B, L, C), flush=True)
    r = blc_and_reference(sc, v, g)
    rows = np.array([0, 1023, 1024, 1099, 1100 + 5, 2 * 1100 - 1])
    ref, S = oracle.causal_conv_f64(v.reshape(-1, L)[rows], g.reshape(-1, L)[rows])
    assert_within_bound(r.reshape(-1, L)[rows], ref, S, False, "blc channel blocks")


def test_medium_shape_bf16(sc):
    w = WORKLOADS[3]
    v, g = make_inputs(w)
    print("case blc medium full shape", flush=True)
    r = blc_and_reference(sc, v, g)
    rows = np.array([0, 1, 1023, 1024, 4097, 8191])
    ref, S = oracle.causal_conv_f64(v.reshape(-1, w.L)[rows], g.reshape(-1, w.L)[rows])
    assert_within_bound(r.reshape(-1, w.L)[rows], ref, S, True, "blc medium")


def test_caller_workspace_and_head_option(sc):
    v, g = make_inputs(WORKLOADS[2], B=3, C=40, L=500, seed_offset=9)
    nbytes = sc.sc_blc_workspace_bytes(sc.KIND_F32, 3, 500, 40)
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda:0")
    a = to_host(sc.causal_conv_blc(to_device(token_major(v)), to_device(token_major(g)),
                                   workspace=ws))
    b = to_host(sc.causal_conv_blc(to_device(token_major(v)), to_device(token_major(g))))
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
    # options pass through: a forced path and head agree with the channel-major call
    print("case blc options", flush=True)
    r = blc_and_reference(sc, v, g, path=sc.PATH_FUSED, head=8)
    ref, S = oracle.causal_conv_f64(v, g)
    assert_within_bound(r, ref, S, False, "blc options")


def test_ordering_on_a_side_stream(sc):
    # several chunks (two per batch row of 9 M elements) on a non-default stream: the call's
    # result is complete for the next work on that stream, without a host synchronisation,
    # and its inputs may be overwritten by that work
    B, L, C = 3, 4096, 2200
    v, g = make_inputs(WORKLOADS[2], B=B, C=C, L=L, seed_offset=77)
    vd, gd = to_device(token_major(v)), to_device(token_major(g))
    ref = to_host(sc.causal_conv_blc(vd, gd))
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    print("case blc side stream", flush=True)
    with torch.cuda.stream(side):
        r = sc.causal_conv_blc(vd, gd)
        twice = r * 2
        vd.zero_()
    torch.cuda.current_stream().wait_stream(side)
    assert np.array_equal(to_host(r).view(np.uint32), ref.view(np.uint32))
    assert np.array_equal(to_host(twice), ref * 2)


def test_fixed_kind_bit_exact(sc):
    # the exact real-valued kind through the token-major call: bit for bit the oracle's
    # fixed-point result (fraction bits 24 and 24)
    import ctypes
    B, L, C = 2, 1000, 70
    v, g = make_inputs(WORKLOADS[2], B=B, C=C, L=L, seed_offset=91)
    opt = sc.sc_options(sc.PATH_AUTO, -1, 24, 24)
    vt, gt = to_device(token_major(v)), to_device(token_major(g))
    r = torch.empty_like(vt)
    print("case blc fixed kind", flush=True)
    st = sc.sc_causal_conv_blc_ex(sc.KIND_FIXED_F32, vt.data_ptr(), gt.data_ptr(), r.data_ptr(),
                                  B, L, C, ctypes.byref(opt), None, 0,
                                  torch.cuda.current_stream().cuda_stream)
    assert st == sc.SC_OK, sc.sc_status_string(st)
    got = np.ascontiguousarray(np.swapaxes(to_host(r), 1, 2))
    ref = oracle.causal_conv_fixed_f32(v, g, 24, 24)
    assert np.array_equal(got.view(np.uint32), ref.astype(np.float32).view(np.uint32))
