"""GPU parity of the gradient calls (backward pass) against the float64 / int64 oracle.

dv_j = sum_{t>=j} dr_t g_{t-j} and dg_k = sum_{t>=k} dr_t v_{t-k} (the vector-Jacobian
product of the causal convolution; the pages' models are trained end to end, "Caracal",
loss function / training strategy).  Float kinds: per output, |d - d_ref| <= 1e-4 * S with
S the oracle's sum of absolute products (plus one bf16 rounding for bf16 storage).  Exact
kind: bit for bit, and dv_j, dg_j do not change when dr_s changes for s < j.
"""
import numpy as np
import pytest
import torch

import oracle
from tests.gpu_util import assert_within_bound, to_device, to_host
from workloads import WORKLOADS, make_grad, make_inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def sc():
    import fft_causal_long_amd as m
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return m


def run(sc, dr, v, g, **kw):
    dv, dg = sc.causal_conv_bwd(to_device(dr), to_device(v), to_device(g), **kw)
    torch.cuda.synchronize()
    return to_host(dv), to_host(dg)


def check(sc, cid, B, C, L, what, seed=0, chans=None, **kw):
    w = WORKLOADS[cid]
    v, g = make_inputs(w, B=B, C=C, L=L, seed_offset=seed)
    dr = make_grad(w, B=B, C=C, L=L, seed_offset=seed)
    print("case %s: B=%d C=%d L=%d %s" % (what, B, C, L, kw), flush=True)
    dv, dg = run(sc, dr, v, g, **kw)
    if chans is not None:
        dr, v, g, dv, dg = [x.reshape(-1, L)[chans] for x in (dr, v, g, dv, dg)]
    rv, rg, Sv, Sg = oracle.causal_conv_bwd_f64(dr, v, g)
    bf16 = v.dtype == np.uint16
    a = assert_within_bound(dv, rv, Sv, bf16, what + " dv")
    b = assert_within_bound(dg, rg, Sg, bf16, what + " dg")
    print("%s: worst err/bound dv %.3g dg %.3g" % (what, a, b), flush=True)


@pytest.mark.parametrize("L", [1, 2, 7, 31, 32])
def test_direct_lengths(sc, L):
    check(sc, 1, 2, 5, L, "direct L=%d" % L, seed=L)


@pytest.mark.parametrize("L", [33, 64, 100, 256, 1000, 1024, 1500, 2048, 2049, 3000, 4095, 4096])
def test_fused_f32(sc, L):
    check(sc, 2, 1, 16, L, "fused f32 L=%d" % L, seed=L)


@pytest.mark.parametrize("L", [64, 1000, 2000, 4096])
def test_fused_bf16(sc, L):
    check(sc, 3, 1, 8, L, "fused bf16 L=%d" % L, seed=L)


def test_fused_ragged_channels_and_head_options(sc):
    # channel counts that leave a workgroup partly empty; head off and at its maximum
    check(sc, 2, 3, 5, 512, "ragged channels", seed=3)
    check(sc, 2, 1, 7, 1024, "head 64", seed=4, head=64)


@pytest.mark.parametrize("L", [2049, 3000, 4096])
def test_four_step_forced(sc, L):
    check(sc, 4, 1, 4, L, "four-step forced L=%d" % L, seed=L, path=sc.PATH_FOUR_STEP)


@pytest.mark.parametrize("L", [4097, 8192, 16384])
def test_four_step_auto(sc, L):
    check(sc, 4, 1, 4, L, "four-step L=%d" % L, seed=L)


def test_four_step_bf16_and_odd_length(sc):
    check(sc, 3, 1, 4, 8192, "four-step bf16 L=8192", seed=21)
    check(sc, 4, 1, 3, 5001, "four-step odd L=5001", seed=22)


def test_four_step_several_chunks(sc):
    L = 16384
    per = sc.sc_workspace_bytes(sc.KIND_F32, 1, 1, L)
    chunk = sc.sc_workspace_bytes(sc.KIND_F32, 1, 10**6, L) // per
    C = chunk + 5
    chans = np.array([0, chunk - 1, chunk, C - 1])
    check(sc, 4, 1, C, L, "four-step %d channels (chunk %d)" % (C, chunk), seed=23, chans=chans)


def test_caller_workspace_matches(sc):
    w = WORKLOADS[4]
    L = 8192
    v, g = make_inputs(w, B=1, C=8, L=L, seed_offset=24)
    dr = make_grad(w, B=1, C=8, L=L, seed_offset=24)
    need = sc.sc_workspace_bytes(sc.KIND_F32, 1, 8, L)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda:0")
    a = sc.causal_conv_bwd(to_device(dr), to_device(v), to_device(g), workspace=ws)
    b = sc.causal_conv_bwd(to_device(dr), to_device(v), to_device(g))
    torch.cuda.synchronize()
    assert torch.equal(a[0].view(torch.int32), b[0].view(torch.int32))
    assert torch.equal(a[1].view(torch.int32), b[1].view(torch.int32))
    small = torch.empty(need - 256, dtype=torch.uint8, device="cuda:0")
    with pytest.raises(sc.SpecConvError) as ei:
        sc.causal_conv_bwd(to_device(dr), to_device(v), to_device(g), workspace=small)
    assert ei.value.status == sc.SC_ERR_WORKSPACE


def test_medium_bf16_full_shape_sampled(sc):
    # the headline shape, all 8192 channels through the kernel; 6 channels checked
    w = WORKLOADS[3]
    check(sc, 3, w.B, w.C, w.L, "medium bf16 full", chans=np.array([0, 1, 1023, 4096, 8190, 8191]))


def test_long_full_shape_sampled(sc):
    w = WORKLOADS[4]
    check(sc, 4, w.B, w.C, w.L, "long f32 full", chans=np.array([0, 700, w.C - 1]))


def test_deterministic(sc):
    w = WORKLOADS[2]
    v, g = make_inputs(w, B=1, C=64, L=1024, seed_offset=30)
    dr = make_grad(w, B=1, C=64, L=1024, seed_offset=30)
    a = run(sc, dr, v, g)
    b = run(sc, dr, v, g)
    assert all(np.array_equal(x.view(np.uint32), y.view(np.uint32)) for x, y in zip(a, b))


# ---------------------------------------------------------------- exact kind

def ntt_case(sc, B, C, L, seed):
    w = WORKLOADS[5]
    v, g = make_inputs(w, B=B, C=C, L=L, seed_offset=seed)
    dr = make_grad(w, B=B, C=C, L=L, seed_offset=seed)
    print("case ntt bwd: B=%d C=%d L=%d" % (B, C, L), flush=True)
    return dr, v, g


@pytest.mark.parametrize("L", [1, 33, 64, 1000, 3000, 4096])
def test_ntt_bit_exact(sc, L):
    dr, v, g = ntt_case(sc, 1, 12, L, seed=L)
    dv, dg = run(sc, dr, v, g)
    rv, rg = oracle.causal_conv_bwd_i64(dr, v, g)
    assert np.abs(rv).max() <= (oracle.P_NTT - 1) // 2
    assert np.array_equal(dv.astype(np.int64), rv)
    assert np.array_equal(dg.astype(np.int64), rg)


def test_ntt_full_shape_sampled(sc):
    w = WORKLOADS[5]
    dr, v, g = ntt_case(sc, w.B, w.C, w.L, seed=0)
    dv, dg = run(sc, dr, v, g)
    ch = np.array([0, 1, 1500, w.B * w.C - 1])
    rv, rg = oracle.causal_conv_bwd_i64(*[x.reshape(-1, w.L)[ch] for x in (dr, v, g)])
    assert np.array_equal(dv.reshape(-1, w.L)[ch].astype(np.int64), rv)
    assert np.array_equal(dg.reshape(-1, w.L)[ch].astype(np.int64), rg)


def test_ntt_gradient_ignores_earlier_output_gradients(sc):
    # dv_j, dg_j read dr_t for t >= j only: changing dr_s leaves j > s bitwise unchanged
    L = 4096
    dr, v, g = ntt_case(sc, 1, 4, L, seed=40)
    base = run(sc, dr, v, g)
    for s in (0, 1, 2047, L - 2):
        d2 = dr.copy()
        d2[..., s] = np.where(d2[..., s] == 5, 6, 5)
        pert = run(sc, d2, v, g)
        for a, b in zip(base, pert):
            assert np.array_equal(a[..., s + 1:], b[..., s + 1:]), s
