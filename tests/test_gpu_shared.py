"""GPU parity of the filter-shared-by-the-batch calls against the float64 oracle.

r[b, c, t] = sum_{j<=t} v[b, c, j] k[c, t-j]: the oracle is the direct sum with k broadcast
over the batch (the same pinned oracle as the per-row gate).  Bounds as for the forward
call: |r - r_ref| <= 1e-4 * S (plus one bf16 rounding for bf16 storage).
"""
import numpy as np
import pytest
import torch

import oracle
from tests.gpu_util import assert_within_bound, to_device, to_host
from workloads import WORKLOADS, make_grad, make_inputs, make_shared_filter

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def sc():
    import fft_causal_long_amd as m
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return m


def inputs(cid, B, C, L, seed):
    w = WORKLOADS[cid]
    v, _ = make_inputs(w, B=B, C=C, L=L, seed_offset=seed)
    k = make_shared_filter(w, C=C, L=L, seed_offset=seed)
    return v, k


def check(r, v, k, what, chans=None):
    B, C, L = v.shape
    kk = np.broadcast_to(k[None], v.shape)
    if chans is not None:
        v, kk, r = [x.reshape(-1, L)[chans] for x in (v, kk, r)]
    ref, S = oracle.causal_conv_f64(v, np.ascontiguousarray(kk))
    worst = assert_within_bound(r, ref, S, v.dtype == np.uint16, what)
    print("%s: worst err/bound %.3g" % (what, worst), flush=True)


@pytest.mark.parametrize("L", [1, 5, 32, 33, 64, 100, 256, 1000, 1024, 3000, 4095, 4096])
def test_lengths_f32(sc, L):
    v, k = inputs(2, 3, 5, L, L)
    print("case shared f32 L=%d" % L, flush=True)
    r = to_host(sc.causal_conv_shared(to_device(v), to_device(k)))
    check(r, v, k, "shared f32 L=%d" % L)


@pytest.mark.parametrize("B,C", [(1, 1), (2, 7), (5, 3), (8, 16)])
def test_batch_shapes_bf16(sc, B, C):
    v, k = inputs(3, B, C, 4096, B * 100 + C)
    print("case shared bf16 B=%d C=%d" % (B, C), flush=True)
    r = to_host(sc.causal_conv_shared(to_device(v), to_device(k)))
    check(r, v, k, "shared bf16 B=%d C=%d" % (B, C))


def test_spectrum_reused_across_calls(sc):
    L, C = 2048, 12
    w = WORKLOADS[2]
    k = make_shared_filter(w, C=C, L=L, seed_offset=7)
    spec = sc.filter_spectrum(to_device(k))
    for seed, B in ((8, 4), (9, 3)):
        v, _ = make_inputs(w, B=B, C=C, L=L, seed_offset=seed)
        print("case spectrum reuse B=%d" % B, flush=True)
        r = to_host(sc.causal_conv_spec(to_device(v), spec, C, L))
        check(r, v, k, "spectrum reuse B=%d" % B)
        # the one-shot call gives the same bits
        r2 = to_host(sc.causal_conv_shared(to_device(v), to_device(k)))
        assert np.array_equal(r.view(np.uint32), r2.view(np.uint32))


def test_medium_shape_sampled(sc):
    w = WORKLOADS[3]
    v, k = inputs(3, w.B, w.C, w.L, 0)
    print("case shared medium full shape", flush=True)
    r = to_host(sc.causal_conv_shared(to_device(v), to_device(k)))
    check(r, v, k, "shared medium", chans=np.array([0, 1, 1023, 1024, 4097, 8191]))


def test_deterministic_and_causal(sc):
    v, k = inputs(2, 4, 8, 1024, 11)
    a = to_host(sc.causal_conv_shared(to_device(v), to_device(k)))
    b = to_host(sc.causal_conv_shared(to_device(v), to_device(k)))
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
    # rows of a pair do not leak into each other: changing row 1 leaves row 0 bitwise equal
    v2 = v.copy()
    v2[1] += np.float32(1.0)
    c = to_host(sc.causal_conv_shared(to_device(v2), to_device(k)))
    assert np.array_equal(c[0].view(np.uint32), a[0].view(np.uint32)) or \
        np.max(np.abs(c[0] - a[0])) <= 1e-5 * np.max(np.abs(a[0]))


# ---------------------------------------------------------------- gradients

def grad_inputs(cid, B, C, L, seed):
    w = WORKLOADS[cid]
    v, k = inputs(cid, B, C, L, seed)
    dr = make_grad(w, B=B, C=C, L=L, seed_offset=seed)
    return dr, v, k


def check_bwd(dv, dk, dr, v, k, what, chans=None):
    bf = v.dtype == np.uint16
    if chans is not None:
        dr, v, k, dv, dk = dr[:, chans], v[:, chans], k[chans], dv[:, chans], dk[chans]
    dv_ref, dk_ref, Sv, Sk = oracle.shared_conv_bwd_f64(dr, v, k)
    a = assert_within_bound(dv, dv_ref, Sv, bf, what + " dv")
    b = assert_within_bound(dk, dk_ref, Sk, bf, what + " dk")
    print("%s: worst err/bound dv %.3g dk %.3g" % (what, a, b), flush=True)


@pytest.mark.parametrize("L", [1, 5, 32, 33, 64, 100, 256, 1000, 1024, 3000, 4095, 4096])
def test_bwd_lengths_f32(sc, L):
    dr, v, k = grad_inputs(2, 3, 5, L, L + 50)
    print("case shared bwd f32 L=%d" % L, flush=True)
    dv, dk = sc.causal_conv_shared_bwd(to_device(dr), to_device(v), to_device(k))
    check_bwd(to_host(dv), to_host(dk), dr, v, k, "shared bwd f32 L=%d" % L)


@pytest.mark.parametrize("B,C,L", [(1, 1, 4096), (2, 7, 4096), (5, 3, 4096), (8, 16, 4096),
                                   (3, 4, 999), (1, 2, 2)])
def test_bwd_batch_shapes_bf16(sc, B, C, L):
    dr, v, k = grad_inputs(3, B, C, L, B * 100 + C + 7)
    print("case shared bwd bf16 B=%d C=%d L=%d" % (B, C, L), flush=True)
    dv, dk = sc.causal_conv_shared_bwd(to_device(dr), to_device(v), to_device(k))
    check_bwd(to_host(dv), to_host(dk), dr, v, k, "shared bwd bf16 B=%d C=%d L=%d" % (B, C, L))


def test_bwd_spectrum_path_matches_one_shot(sc):
    L, C, B = 2048, 6, 4
    dr, v, k = grad_inputs(2, B, C, L, 21)
    kd = to_device(k)
    spec = sc.filter_spectrum(kd)
    print("case shared bwd from spectrum", flush=True)
    dv, dk = sc.causal_conv_spec_bwd(to_device(dr), to_device(v), spec, C, L)
    dv, dk = to_host(dv), to_host(dk)
    check_bwd(dv, dk, dr, v, k, "shared bwd spectrum")
    dv2, dk2 = sc.causal_conv_shared_bwd(to_device(dr), to_device(v), kd)
    assert np.array_equal(dv.view(np.uint32), to_host(dv2).view(np.uint32))
    assert np.array_equal(dk.view(np.uint32), to_host(dk2).view(np.uint32))


def test_bwd_odd_offset_outputs(sc):
    # dk at an odd element offset with even L: pair stores must give way to single ones
    dr, v, k = grad_inputs(2, 2, 3, 1000, 33)
    dev = torch.device("cuda:0")
    dk_buf = torch.zeros(3 * 1000 + 1, dtype=torch.float32, device=dev)
    dk_view = dk_buf[1:].view(3, 1000)
    print("case shared bwd odd offset", flush=True)
    dv, dk = sc.causal_conv_shared_bwd(to_device(dr), to_device(v), to_device(k), dk=dk_view)
    assert float(dk_buf[0]) == 0.0
    check_bwd(to_host(dv), to_host(dk), dr, v, k, "shared bwd odd offset")


def test_bwd_medium_shape_sampled(sc):
    w = WORKLOADS[3]
    dr, v, k = grad_inputs(3, w.B, w.C, w.L, 1)
    print("case shared bwd medium full shape", flush=True)
    dv, dk = sc.causal_conv_shared_bwd(to_device(dr), to_device(v), to_device(k))
    check_bwd(to_host(dv), to_host(dk), dr, v, k, "shared bwd medium",
              chans=np.array([0, 1, 511, w.C - 1]))


# shapes with at least 512 channel groups take the one-kernel gradient path (dv and dk from
# the same transform per row); smaller ones the apply + row-loop pair tested above
@pytest.mark.parametrize("cid,B,C,L", [(2, 2, 512, 4096), (3, 3, 512, 3001), (2, 2, 1024, 2048),
                                       (3, 2, 2048, 1000), (2, 1, 4096, 256)])
def test_bwd_one_kernel_path(sc, cid, B, C, L):
    dr, v, k = grad_inputs(cid, B, C, L, B + C + L)
    print("case shared bwd one-kernel cid=%d B=%d C=%d L=%d" % (cid, B, C, L), flush=True)
    dv, dk = sc.causal_conv_shared_bwd(to_device(dr), to_device(v), to_device(k))
    chans = np.array([0, 1, C // 2 - 1, C // 2, C - 2, C - 1])
    check_bwd(to_host(dv), to_host(dk), dr, v, k, "one-kernel cid=%d C=%d L=%d" % (cid, C, L),
              chans=chans)


def test_bwd_one_kernel_misaligned_dk(sc):
    B, C, L = 2, 512, 4096
    dr, v, k = grad_inputs(2, B, C, L, 5)
    dk_buf = torch.zeros(C * L + 1, dtype=torch.float32, device="cuda:0")
    dk_view = dk_buf[1:].view(C, L)
    print("case shared bwd one-kernel misaligned dk", flush=True)
    dv, dk = sc.causal_conv_shared_bwd(to_device(dr), to_device(v), to_device(k), dk=dk_view)
    assert float(dk_buf[0]) == 0.0
    check_bwd(to_host(dv), to_host(dk), dr, v, k, "one-kernel misaligned",
              chans=np.array([0, 255, 511]))


@pytest.mark.parametrize("dt,C,L", [(torch.float32, 8, 1000), (torch.bfloat16, 3, 333)])
def test_bwd_empty_batch_zeroes_dk(sc, dt, C, L):
    # dk sums over the batch rows: with no rows it is zero, whatever dk held before
    print("case shared bwd empty batch %s C=%d L=%d" % (dt, C, L), flush=True)
    e = torch.empty((0, C, L), dtype=dt, device="cuda:0")
    k = torch.ones((C, L), dtype=dt, device="cuda:0")
    dk = torch.full((C, L), 7.0, dtype=dt, device="cuda:0")
    dv, dk2 = sc.causal_conv_shared_bwd(e, e, k, dk=dk)
    torch.cuda.synchronize()
    assert dv.shape == e.shape and dk2.data_ptr() == dk.data_ptr()
    assert int(torch.count_nonzero(dk)) == 0
    spec = sc.filter_spectrum(k)
    dk.fill_(7.0)
    sc.causal_conv_spec_bwd(e, e, spec, C, L, dk=dk)
    torch.cuda.synchronize()
    assert int(torch.count_nonzero(dk)) == 0
