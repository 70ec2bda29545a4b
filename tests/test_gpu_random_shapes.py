"""GPU parity on seeded random shapes: every float kind and path the automatic choice
takes (direct, fused, four-step), forward and gradients, and the exact kinds (int32 NTT
with its gradients, the real-valued fixed-point kind) bit for bit, at lengths drawn
log-uniformly over 1 .. 9000 and channel counts that leave partial workgroups.  The bounds are those of the fixed-shape tests (tests/gpu_util.py)."""
import numpy as np
import pytest
import torch

import oracle
from tests.gpu_util import assert_within_bound, to_device, to_host
from workloads import WORKLOADS, make_inputs

pytestmark = pytest.mark.gpu

_rng = np.random.default_rng(20261203)
SHAPES = []
for _ in range(16):
    L = int(np.exp(_rng.uniform(0.0, np.log(9000.0))))
    B = int(_rng.integers(1, 4))
    C = int(_rng.integers(1, 40))
    SHAPES.append((B, C, max(L, 1)))


@pytest.fixture(scope="module")
def sc():
    import fft_causal_long_amd as m
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return m


@pytest.mark.parametrize("i", range(len(SHAPES)))
def test_random_shape_float_forward_and_gradients(sc, i):
    B, C, L = SHAPES[i]
    cid = 4 if i % 2 == 0 else 3                  # fp32 (long-context recipe) or bf16
    v, g = make_inputs(WORKLOADS[cid], B=B, C=C, L=L, seed_offset=300 + i)
    dr, _ = make_inputs(WORKLOADS[cid], B=B, C=C, L=L, seed_offset=400 + i)
    bf = v.dtype == np.uint16
    what = "random %d: B=%d C=%d L=%d %s" % (i, B, C, L, "bf16" if bf else "f32")
    print("case " + what, flush=True)
    tv, tg, td = to_device(v), to_device(g), to_device(dr)
    r = to_host(sc.causal_conv(tv, tg))
    dv, dg = sc.causal_conv_bwd(td, tv, tg)
    torch.cuda.synchronize()
    r_ref, S = oracle.causal_conv_f64(v, g)
    assert_within_bound(r, r_ref, S, bf, what)
    dv_ref, dg_ref, Sv, Sg = oracle.causal_conv_bwd_f64(dr, v, g)
    assert_within_bound(to_host(dv), dv_ref, Sv, bf, what + " dv")
    assert_within_bound(to_host(dg), dg_ref, Sg, bf, what + " dg")


@pytest.mark.parametrize("i", range(len(SHAPES)))
def test_random_shape_exact(sc, i):
    # fused up to L = 4096, the four-step split beyond; forward and gradients bit for bit
    B, C, L = SHAPES[i]
    v, g = make_inputs(WORKLOADS[5], B=B, C=C, L=L, seed_offset=500 + i)
    dr, _ = make_inputs(WORKLOADS[5], B=B, C=C, L=L, seed_offset=700 + i)
    print("case random exact %d: B=%d C=%d L=%d" % (i, B, C, L), flush=True)
    tv, tg = to_device(v), to_device(g)
    r = to_host(sc.causal_conv(tv, tg))
    dv, dg = sc.causal_conv_bwd(to_device(dr), tv, tg)
    torch.cuda.synchronize()
    assert np.array_equal(r.astype(np.int64), oracle.lift_mod_p(oracle.causal_conv_i64(v, g)))
    rdv, rdg = oracle.causal_conv_bwd_i64(dr, v, g)
    assert np.array_equal(to_host(dv).astype(np.int64), oracle.lift_mod_p(rdv))
    assert np.array_equal(to_host(dg).astype(np.int64), oracle.lift_mod_p(rdg))


@pytest.mark.parametrize("i", range(0, len(SHAPES), 2))
def test_random_shape_token_major(sc, i):
    # the (B, L, C) call gives the bits of the channel-major call on the transposed tensors
    B, C, L = SHAPES[i]
    v, g = make_inputs(WORKLOADS[3], B=B, C=C, L=L, seed_offset=600 + i)
    print("case random token-major %d: B=%d C=%d L=%d" % (i, B, C, L), flush=True)
    tv, tg = to_device(v), to_device(g)
    r_cm = sc.causal_conv(tv, tg)
    r_tm = sc.causal_conv_blc(tv.transpose(1, 2).contiguous(), tg.transpose(1, 2).contiguous())
    torch.cuda.synchronize()
    assert torch.equal(r_tm.transpose(1, 2).contiguous().view(torch.int16), r_cm.view(torch.int16))


@pytest.mark.parametrize("i", range(1, len(SHAPES), 4))
def test_random_shape_gate_mixing_step(sc, i):
    # channel counts rounded up to whole gate groups; both layouts give the bits of the gate
    # call followed by the convolution
    from workloads import make_gate_inputs
    B, C, L = SHAPES[i]
    C = 64 * ((C + 63) // 64)
    v, s, W = make_gate_inputs(WORKLOADS[3], B=B, C=C, L=L, seed_offset=700 + i)
    print("case random gate %d: B=%d C=%d L=%d" % (i, B, C, L), flush=True)
    tv, ts, tW = to_device(v), to_device(s), to_device(W)
    g = sc.gate(ts, tW)
    r_sep = sc.causal_conv(tv, g)
    r_cm = sc.gate_conv(tv, ts, tW)
    r_tm = sc.gate_conv_blc(tv.transpose(1, 2).contiguous(), ts.transpose(1, 2).contiguous(), tW)
    torch.cuda.synchronize()
    assert torch.equal(r_cm.view(torch.int16), r_sep.view(torch.int16))
    assert torch.equal(r_tm.transpose(1, 2).contiguous().view(torch.int16), r_sep.view(torch.int16))


@pytest.mark.parametrize("i", [i for i in range(len(SHAPES)) if SHAPES[i][2] <= 4096 and i % 3 == 0])
def test_random_shape_shared_filter(sc, i):
    # one filter per channel shared by the batch: forward and both gradients (dk summed
    # over the batch) against the oracle's bounds
    from workloads import make_grad, make_shared_filter
    B, C, L = SHAPES[i]
    w = WORKLOADS[4 if i % 2 == 0 else 3]
    v, _ = make_inputs(w, B=B, C=C, L=L, seed_offset=800 + i)
    k = make_shared_filter(w, C=C, L=L, seed_offset=800 + i)
    dr = make_grad(w, B=B, C=C, L=L, seed_offset=900 + i)
    bf = v.dtype == np.uint16
    what = "random shared %d: B=%d C=%d L=%d %s" % (i, B, C, L, "bf16" if bf else "f32")
    print("case " + what, flush=True)
    tv, tk, td = to_device(v), to_device(k), to_device(dr)
    r = to_host(sc.causal_conv_shared(tv, tk))
    dv, dk = sc.causal_conv_shared_bwd(td, tv, tk)
    torch.cuda.synchronize()
    r_ref, S = oracle.causal_conv_f64(v, np.ascontiguousarray(np.broadcast_to(k[None], v.shape)))
    assert_within_bound(r, r_ref, S, bf, what)
    dv_ref, dk_ref, Sv, Sk = oracle.shared_conv_bwd_f64(dr, v, k)
    assert_within_bound(to_host(dv), dv_ref, Sv, bf, what + " dv")
    assert_within_bound(to_host(dk), dk_ref, Sk, bf, what + " dk")


@pytest.mark.parametrize("i", [i for i in range(len(SHAPES)) if i % 3 == 1 or SHAPES[i][2] > 4096])
def test_random_shape_exact_real_valued(sc, i):
    # fixed-point encoding with 20 + 20 fraction bits, three primes (fused, or the four-step
    # split beyond L = 4096): bit for bit the oracle
    B, C, L = SHAPES[i]
    v, g = make_inputs(WORKLOADS[4], B=B, C=C, L=L, seed_offset=1000 + i)
    assert sc.sc_fixed_range_ok(float(np.abs(v).max()), float(np.abs(g).max()), 20, 20, L)
    print("case random exact real-valued %d: B=%d C=%d L=%d" % (i, B, C, L), flush=True)
    r = to_host(sc.causal_conv_fixed(to_device(v), to_device(g), 20, 20))
    torch.cuda.synchronize()
    ref = oracle.causal_conv_fixed_f32(v, g, 20, 20)
    assert np.array_equal(r.view(np.uint32), ref.view(np.uint32))
