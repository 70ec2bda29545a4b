"""GPU parity of the exactly causal real-valued path (sc_causal_conv_fixed_f32) against the
oracle, bit for bit.

The definition: V = round(v 2^fv), G = round(g 2^fg) (nearest, ties to even), R the exact
integer causal sum, r = R 2^-(fv+fg) rounded once to float32.  The oracle computes R by
direct 128-bit summation and rounds with Python integers; the library computes R modulo
three primes and combines them (Chinese remainder theorem), so every output must match
bit for bit, and no output may move when a later input changes ("Catastrophic Token
Leakage ...", abstract: integer transforms leak nothing).
"""
import numpy as np
import pytest
import torch

import oracle
from tests.gpu_util import to_device, to_host
from workloads import WORKLOADS, make_inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def sc():
    import fft_causal_long_amd as m
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return m


def run(sc, v, g, fv, fg, **kw):
    out = sc.causal_conv_fixed(to_device(v), to_device(g), fv, fg, **kw)
    torch.cuda.synchronize()
    return to_host(out)


def check(sc, v, g, fv, fg, what, chans=None):
    L = v.shape[-1]
    amax_v, amax_g = float(np.abs(v).max()), float(np.abs(g).max())
    assert sc.sc_fixed_range_ok(amax_v, amax_g, fv, fg, L), what
    print("case %s: shape %s fv=%d fg=%d" % (what, v.shape, fv, fg), flush=True)
    r = run(sc, v, g, fv, fg)
    if chans is not None:
        v, g, r = [x.reshape(-1, L)[chans] for x in (v, g, r)]
    ref = oracle.causal_conv_fixed_f32(v, g, fv, fg)
    diff = r.view(np.uint32) != ref.view(np.uint32)
    assert not diff.any(), "%s: %d of %d outputs differ; first at %s (gpu %r, ref %r)" % (
        what, int(diff.sum()), diff.size, np.argwhere(diff)[0], r[diff][0], ref[diff][0])


@pytest.mark.parametrize("L", [1, 2, 33, 64, 100, 128, 200, 256, 257, 513, 1000, 2048, 3000, 4095, 4096])
def test_lengths_bit_exact(sc, L):
    v, g = make_inputs(WORKLOADS[2], B=1, C=6, L=L, seed_offset=L)
    check(sc, v, g, 24, 24, "L=%d" % L)


@pytest.mark.parametrize("fv,fg", [(0, 0), (8, 30), (30, 8), (-3, 40), (36, 36)])
def test_fraction_bits(sc, fv, fg):
    # wide fraction ranges push R towards 2^80 and exercise all three residues
    rng = np.random.default_rng((fv + 100) * 1000 + fg)
    L = 1024
    v = rng.standard_normal((1, 4, L)).astype(np.float32)
    g = rng.standard_normal((1, 4, L)).astype(np.float32)
    if fv + fg > 60:
        v *= np.float32(2.0 ** -4)
        g *= np.float32(2.0 ** -4)
    if fv == 0:
        v *= np.float32(1000.0)
        g *= np.float32(1000.0)
    check(sc, v, g, fv, fg, "fv=%d fg=%d" % (fv, fg))


def test_near_the_exact_range(sc):
    # |R| close to (p_A p_B p_C - 1)/2: encodings near 2^43.5 with L = 1
    v = np.array([[[2.0 ** 43.5]]], dtype=np.float32)
    g = np.array([[[-2.0 ** 43.6]]], dtype=np.float32)
    check(sc, v, g, 0, 0, "near range")
    rng = np.random.default_rng(7)
    v = (rng.uniform(-1, 1, (1, 2, 64)) * 2.0 ** 38).astype(np.float32)
    g = (rng.uniform(-1, 1, (1, 2, 64)) * 2.0 ** 38).astype(np.float32)
    check(sc, v, g, 0, 0, "large encodings L=64")


def test_subnormal_and_tiny_results(sc):
    rng = np.random.default_rng(8)
    v = rng.integers(-3, 4, (1, 2, 64)).astype(np.float32)
    g = rng.integers(-3, 4, (1, 2, 64)).astype(np.float32)
    # encodings V = v 2^64 are the small integers themselves, so r = R 2^-128 falls below
    # the smallest normal float32 (2^-126) for |R| < 4
    check(sc, v * np.float32(2.0 ** -64), g * np.float32(2.0 ** -64), 64, 64, "tiny")


@pytest.mark.parametrize("fv,fg", [(0, 0), (10, 6)])
def test_exact_ties_round_to_even(sc, fv, fg):
    # r_1 = R_0 + x with R_0 = 2^24 or 2^25: float32 spacing 2 or 4 there, so odd x (resp.
    # x = 2 mod 4) lands exactly halfway between two floats and must go to the even one
    base = [2.0 ** 24, 2.0 ** 24, 2.0 ** 24, 2.0 ** 24, 2.0 ** 25, 2.0 ** 25, -2.0 ** 24, -2.0 ** 24]
    xs = [1.0, 3.0, 5.0, -1.0, 2.0, 6.0, -1.0, -3.0]
    want = [2.0 ** 24, 2.0 ** 24 + 4, 2.0 ** 24 + 4, 2.0 ** 24 - 1, 2.0 ** 25, 2.0 ** 25 + 8,
            -2.0 ** 24, -(2.0 ** 24 + 4)]
    n = len(base)
    v = np.zeros((1, n, 2), np.float32)
    g = np.zeros((1, n, 2), np.float32)
    v[0, :, 0] = np.array(base) * 2.0 ** -fv
    v[0, :, 1] = np.array(xs) * 2.0 ** -fv
    g[0, :, :] = 2.0 ** -fg                       # G = (1, 1): R_1 = base + x
    check(sc, v, g, fv, fg, "ties fv=%d fg=%d" % (fv, fg))
    r = run(sc, v, g, fv, fg)
    sc_ = 2.0 ** -(fv + fg)
    assert r[0, :, 0].tolist() == [b_ * sc_ for b_ in base]
    assert r[0, :, 1].tolist() == [w_ * sc_ for w_ in want]


def test_ragged_channels_and_workspace(sc):
    v, g = make_inputs(WORKLOADS[2], B=3, C=5, L=500, seed_offset=9)
    check(sc, v, g, 20, 22, "ragged channels")
    # the kind needs no scratch; a caller workspace is accepted and left unused
    assert sc.sc_workspace_bytes(sc.KIND_FIXED_F32, 3, 5, 500) == 0
    ws = torch.full((4096,), 7, dtype=torch.uint8, device="cuda:0")
    a = sc.causal_conv_fixed(to_device(v), to_device(g), 20, 22, workspace=ws)
    b = sc.causal_conv_fixed(to_device(v), to_device(g), 20, 22)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int32), b.view(torch.int32))
    assert bool((ws == 7).all())


def test_medium_shape_sampled(sc):
    # the Medium channel count at L = 4096 (bf16 data widened to float32)
    w = WORKLOADS[3]
    vb, gb = make_inputs(w)
    v = oracle.bf16_bits_to_f64(vb).astype(np.float32)
    g = oracle.bf16_bits_to_f64(gb).astype(np.float32)
    check(sc, v, g, 24, 24, "medium shape", chans=np.array([0, 4095, 8191]))


def test_exact_causality(sc):
    # changing v_s or g_s leaves every output t < s bitwise unchanged
    L = 4096
    v, g = make_inputs(WORKLOADS[2], B=1, C=4, L=L, seed_offset=10)
    base = run(sc, v, g, 24, 24)
    for s in (1, 1000, L - 1):
        v2, g2 = v.copy(), g.copy()
        v2[..., s] += np.float32(0.5)
        g2[..., s] -= np.float32(0.25)
        r2 = run(sc, v2, g2, 24, 24)
        assert np.array_equal(r2[..., :s].view(np.uint32), base[..., :s].view(np.uint32)), s
        assert not np.array_equal(r2[..., s], base[..., s])
