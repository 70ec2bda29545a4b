"""GPU parity of the gate-stream calls against the float64 oracle.

g = Conv1d_G2(sigmoid(s)) (oracle.gate_f64) with error scale Sg = sum |W| sigmoid(s):
    fp32:  |g - g_ref| <= 1e-4 Sg
    bf16:  |g - g_ref| <= (2^-8 + 1e-4) Sg + 2^-8 (|g_ref| + (2^-8 + 1e-4) Sg)
(bf16 storage rounds each sigmoid to bf16 before the product, relative error <= 2^-8 per
term, then g once).  The mixing step r = causal_conv(v, g) is checked three ways: bit for bit
against the separate calls gate + causal_conv (channel-major and token-major run the same
kernels on the same values); against the oracle's causal sum of v and the GPU's own stored g
(the convolution's bound); and end to end against causal(v, g_ref), with the gate's bound
carried through the sum: |r - r_ref| <= 1e-4 S(v, |g_ref|) + sum_j |v_j| bound_g[t-j] (+ one
bf16 rounding of r).
"""
import numpy as np
import pytest
import torch

import oracle
from tests.gpu_util import TOL, assert_within_bound, decode, to_device, to_host
from workloads import WORKLOADS, make_gate_inputs

pytestmark = pytest.mark.gpu
U8 = 2.0 ** -8


@pytest.fixture(scope="module")
def sc():
    import fft_causal_long_amd as m
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return m


def gate_bound(g_ref, Sg, bf16):
    if not bf16:
        return TOL * Sg
    b = (U8 + TOL) * Sg
    return b + U8 * (np.abs(g_ref) + b)


def check_gate(g, s, W, what):
    bf = s.dtype == np.uint16
    g_ref, Sg = oracle.gate_f64(s, W)
    err = np.abs(decode(g) - g_ref)
    b = gate_bound(g_ref, Sg, bf)
    worst = float(np.max(err / np.maximum(b, 1e-300)))
    print("%s: worst err/bound %.3g" % (what, worst), flush=True)
    assert np.all(err <= b), "%s: %d outside the bound" % (what, int(np.sum(err > b)))
    return g_ref, b


def check_end_to_end(r, v, g_ref, gb, bf16, what):
    ref, S = oracle.causal_conv_f64(v, g_ref)
    prop, _ = oracle.causal_conv_f64(np.abs(oracle.as_f64(v)), gb, with_scale=True)
    b = TOL * S + prop
    if bf16:
        b = b + U8 * (np.abs(ref) + b)
    err = np.abs(decode(r) - ref)
    worst = float(np.max(err / np.maximum(b, 1e-300)))
    print("%s end to end: worst err/bound %.3g" % (what, worst), flush=True)
    assert np.all(err <= b), "%s: %d outside the bound" % (what, int(np.sum(err > b)))


def token_major(x):
    return np.ascontiguousarray(np.swapaxes(x, 1, 2))


def channel_major(x):
    return np.ascontiguousarray(np.swapaxes(x, 1, 2))


@pytest.mark.parametrize("cid", [2, 3])
@pytest.mark.parametrize("B,C,L", [(2, 64, 1), (1, 128, 33), (2, 64, 256), (1, 64, 257),
                                   (3, 192, 1000), (1, 64, 4096)])
def test_gate_against_oracle(sc, cid, B, C, L):
    v, s, W = make_gate_inputs(WORKLOADS[cid], B=B, C=C, L=L, seed_offset=B + C + L)
    print("case gate cid=%d B=%d C=%d L=%d" % (cid, B, C, L), flush=True)
    g = to_host(sc.gate(to_device(s), to_device(W)))
    check_gate(g, s, W, "gate cid=%d B=%d C=%d L=%d" % (cid, B, C, L))


@pytest.mark.parametrize("cid", [2, 3])
@pytest.mark.parametrize("B,C,L", [(2, 64, 100), (1, 128, 1024), (2, 64, 4096), (1, 64, 5000)])
def test_gate_conv_both_layouts(sc, cid, B, C, L):
    v, s, W = make_gate_inputs(WORKLOADS[cid], B=B, C=C, L=L, seed_offset=7 * L + C)
    bf = v.dtype == np.uint16
    what = "gate_conv cid=%d B=%d C=%d L=%d" % (cid, B, C, L)
    print("case " + what, flush=True)
    Wd = to_device(W)
    g = to_host(sc.gate(to_device(s), Wd))
    r_sep = to_host(sc.causal_conv(to_device(v), to_device(g)))
    r_cm = to_host(sc.gate_conv(to_device(v), to_device(s), Wd))
    r_tm = channel_major(to_host(sc.gate_conv_blc(to_device(token_major(v)),
                                                  to_device(token_major(s)), Wd)))
    assert np.array_equal(r_cm.view(np.uint8), r_sep.view(np.uint8)), "channel-major"
    assert np.array_equal(r_tm.view(np.uint8), r_sep.view(np.uint8)), "token-major"
    ref, S = oracle.causal_conv_f64(v, g)
    assert_within_bound(r_cm, ref, S, bf, what)
    g_ref, gb = check_gate(g, s, W, what + " gate")
    check_end_to_end(r_cm, v, g_ref, gb, bf, what)


def test_gate_conv_blc_medium_shape(sc):
    w = WORKLOADS[3]
    v, s, W = make_gate_inputs(w)
    print("case gate_conv_blc medium full shape", flush=True)
    vt, st_ = to_device(token_major(v)), to_device(token_major(s))
    Wd = to_device(W)
    r = channel_major(to_host(sc.gate_conv_blc(vt, st_, Wd)))
    # the same bits as the token-major convolution of the gate's own output
    g = to_host(sc.gate(to_device(s), Wd))
    r2 = channel_major(to_host(sc.causal_conv_blc(vt, to_device(token_major(g)))))
    assert np.array_equal(r.view(np.uint16), r2.view(np.uint16))
    # sampled channels end to end: the oracle's gate over their whole groups
    for b, grp, cl in ((0, 0, 0), (3, 5, 17), (7, 15, 63)):
        cs = slice(64 * grp, 64 * grp + 64)
        g_ref, Sg = oracle.gate_f64(s[b:b + 1, cs], W[cs])
        gb = gate_bound(g_ref, Sg, True)
        check_end_to_end(r[b:b + 1, 64 * grp + cl:64 * grp + cl + 1], v[b:b + 1, 64 * grp + cl:64 * grp + cl + 1],
                         g_ref[:, cl:cl + 1], gb[:, cl:cl + 1], True, "medium b=%d c=%d" % (b, 64 * grp + cl))


def test_gate_workspace_and_deterministic(sc):
    v, s, W = make_gate_inputs(WORKLOADS[2], B=3, C=128, L=700, seed_offset=5)
    nbytes = sc.sc_gate_conv_workspace_bytes(sc.KIND_F32, 3, 128, 700)
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda:0")
    a = to_host(sc.gate_conv(to_device(v), to_device(s), to_device(W), workspace=ws))
    b = to_host(sc.gate_conv(to_device(v), to_device(s), to_device(W)))
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


def test_adjacent_buffers_are_not_overlapping(sc):
    # W placed right after g in one allocation (as a caching allocator may do): the call must
    # accept it and compute the same g
    v, s, W = make_gate_inputs(WORKLOADS[2], B=2, C=64, L=256, seed_offset=41)
    n, wn = s.size, W.size
    buf = torch.empty(n + wn, dtype=torch.float32, device="cuda:0")
    g = buf[:n].view(s.shape)
    Wd = buf[n:].view(W.shape)
    Wd.copy_(to_device(W))
    print("case gate adjacent buffers", flush=True)
    sc.gate(to_device(s), Wd, out=g)
    check_gate(to_host(g), s, W, "gate adjacent")


@pytest.mark.parametrize("L", [256, 1000, 4096])
def test_channel_major_vector_and_element_inputs_agree(sc, L):
    # bf16 rows of a multiple of 8 tokens starting 16-byte aligned go through 16-byte loads
    # and an LDS transpose; s one element off its alignment takes the element loads: both
    # feed the same sigma values to the same products, so g is bit for bit the same
    v, s, W = make_gate_inputs(WORKLOADS[3], B=2, C=128, L=L, seed_offset=L + 3)
    n = s.size
    Wd = to_device(W)
    buf = torch.empty(n + 8, dtype=torch.bfloat16, device="cuda:0")
    s_al = buf[8:8 + n].view(s.shape)
    s_al.copy_(to_device(s))
    s_un = torch.empty(n + 1, dtype=torch.bfloat16, device="cuda:0")[1:].view(s.shape)
    s_un.copy_(to_device(s))
    assert s_al.data_ptr() % 16 == 0 and s_un.data_ptr() % 16 != 0
    print("case gate channel-major aligned/unaligned L=%d" % L, flush=True)
    g_al = to_host(sc.gate(s_al, Wd))
    g_un = to_host(sc.gate(s_un, Wd))
    assert np.array_equal(g_al.view(np.uint16), g_un.view(np.uint16))
    check_gate(g_al, s, W, "gate aligned L=%d" % L)
