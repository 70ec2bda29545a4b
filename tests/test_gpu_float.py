"""GPU parity of the float paths (fp32 and bf16 storage) against the float64 oracle.

Every case calls libspecconv through its C ABI (via the ctypes binding) on seeded
synthetic inputs and compares element by element with the oracle on the same stored
inputs, within the per-output bound of tests/gpu_util.py.
"""
import numpy as np
import pytest
import torch

import oracle
from tests.gpu_util import assert_within_bound, decode, to_device, to_host
from workloads import WORKLOADS, make_inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def sc():
    import fft_causal_long_amd as m
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return m


def run(sc, v, g, **kw):
    tv, tg = to_device(v), to_device(g)
    out = sc.causal_conv(tv, tg, **kw)
    torch.cuda.synchronize()
    return to_host(out)


def check(sc, v, g, what, **kw):
    r = run(sc, v, g, **kw)
    r_ref, S = oracle.causal_conv_f64(v, g)
    worst = assert_within_bound(r, r_ref, S, v.dtype == np.uint16, what)
    print("%s: worst err/bound = %.3g" % (what, worst), flush=True)
    return r, worst


def test_tiny_full(sc):
    v, g = make_inputs(WORKLOADS[1])
    check(sc, v, g, "tiny")


def test_small_full(sc):
    v, g = make_inputs(WORKLOADS[2])
    check(sc, v, g, "small")


LS = [1, 2, 3, 5, 16, 31, 32, 33, 47, 63, 64, 65, 100, 127, 128, 129, 255, 256, 257, 300,
      511, 512, 513, 1000, 1023, 1024, 1025, 2047, 2048, 2049, 3001, 4095, 4096]


@pytest.mark.parametrize("L", LS)
def test_length_sweep_f32(sc, L):
    # 15 channels: not a multiple of the channels-per-workgroup of any small M
    v, g = make_inputs(WORKLOADS[1], B=3, C=5, L=L, seed_offset=L)
    check(sc, v, g, "f32 L=%d" % L)


@pytest.mark.parametrize("L", [33, 64, 257, 1024, 2049, 4096])
def test_length_sweep_bf16_conv_gate(sc, L):
    v, g = make_inputs(WORKLOADS[3], B=2, C=16, L=L, seed_offset=L)
    check(sc, v, g, "bf16 L=%d" % L)


@pytest.mark.parametrize("L", [256, 1024, 4096])
def test_fp32_conv_gate_shapes(sc, L):
    v, g = make_inputs(WORKLOADS[2], B=2, C=64, L=L, seed_offset=7 + L)
    check(sc, v, g, "f32 conv-gate L=%d" % L)


def test_medium_full_size_sampled(sc):
    # full Caracal-Medium shape in the launch configuration the benchmark times; the
    # oracle checks 96 whole channels spread over the batch
    w = WORKLOADS[3]
    v, g = make_inputs(w)
    r = run(sc, v, g)
    nch = w.B * w.C
    chans = np.unique(np.concatenate([[0, nch - 1], np.random.default_rng(3).integers(0, nch, 94)]))
    vs = v.reshape(nch, w.L)[chans]
    gs = g.reshape(nch, w.L)[chans]
    r_ref, S = oracle.causal_conv_f64(vs, gs)
    worst = assert_within_bound(r.reshape(nch, w.L)[chans], r_ref, S, True, "medium sampled")
    print("medium sampled: worst err/bound = %.3g" % worst, flush=True)


def test_medium_shape_as_fp32_sampled(sc):
    w = WORKLOADS[3]
    v, g = make_inputs(w, B=2)
    v32, g32 = decode(v).astype(np.float32), decode(g).astype(np.float32)
    r = run(sc, v32, g32)
    chans = np.arange(0, 2 * w.C, 37)
    r_ref, S = oracle.causal_conv_f64(v32.reshape(-1, w.L)[chans], g32.reshape(-1, w.L)[chans])
    assert_within_bound(r.reshape(-1, w.L)[chans], r_ref, S, False, "medium fp32 sampled")


def test_bitwise_deterministic(sc):
    v, g = make_inputs(WORKLOADS[2], B=1, C=128, L=1024)
    a = run(sc, v, g)
    b = run(sc, v, g)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
    v, g = make_inputs(WORKLOADS[3], B=1, C=64, L=4096)
    a = run(sc, v, g)
    b = run(sc, v, g)
    assert np.array_equal(a, b)


def test_side_stream_and_offsets(sc):
    v, g = make_inputs(WORKLOADS[1], B=1, C=9, L=500)
    r_ref, S = oracle.causal_conv_f64(v, g)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        tv, tg = to_device(v), to_device(g)
        # an output that is 4-byte but not 8-byte aligned (paired stores must be avoided)
        buf = torch.empty(v.size + 1, dtype=torch.float32, device="cuda:0")
        out = buf[1:].view(v.shape)
        sc.causal_conv(tv, tg, out=out)
    s.synchronize()
    assert_within_bound(to_host(out), r_ref, S, False, "side stream, offset output")


def test_paths_agree_with_oracle(sc):
    v, g = make_inputs(WORKLOADS[1], B=1, C=6, L=200, seed_offset=3)
    for path in (sc.PATH_DIRECT, sc.PATH_FUSED):
        check(sc, v, g, "path %d" % path, path=path)
    # fused path for a length the automatic choice sends to direct summation
    v, g = make_inputs(WORKLOADS[1], B=1, C=6, L=20, seed_offset=4)
    check(sc, v, g, "forced fused L=20", path=sc.PATH_FUSED)


@pytest.mark.parametrize("L", [256, 1024])
def test_head_length_option(sc, L):
    v, g = make_inputs(WORKLOADS[1], B=1, C=64, L=L, seed_offset=5)
    r_ref, S = oracle.causal_conv_f64(v, g)
    r0 = run(sc, v, g, head=0)        # every output from the transform
    r64 = run(sc, v, g, head=64)
    assert_within_bound(r64, r_ref, S, False, "head=64")
    # outputs from t = 64 on are the same computation in both runs
    assert np.array_equal(r0[..., 64:], r64[..., 64:])
    # with head = 0 the transform's global round-off is visible at t = 0
    assert np.abs(r0[..., 0] - r_ref[..., 0]).max() > 0.0


def test_empty_is_noop(sc):
    for shape in ((0, 4, 16), (2, 0, 16), (2, 4, 0)):
        t = torch.zeros(shape, dtype=torch.float32, device="cuda:0")
        out = sc.causal_conv(t, t.clone())
        assert out.shape == shape


def test_fp32_leakage_is_small_but_reported(sc):
    # "Catastrophic Token Leakage ..." (abstract): a float FFT convolution lets a change at
    # position s move outputs t < s through round-off.  Measure max_{t<s} |dr_t| with the
    # original and perturbed rows in one launch.
    from workloads import perturbation_positions
    w = WORKLOADS[3]
    L = w.L
    v, g = make_inputs(w, B=1, C=16)
    v32, g32 = decode(v).astype(np.float32), decode(g).astype(np.float32)
    pos = perturbation_positions(w.cid, L)
    vv = np.concatenate([v32] + [v32.copy() for _ in pos], axis=0)
    gg = np.concatenate([g32] * (len(pos) + 1), axis=0)
    for i, s in enumerate(pos):
        vv[i + 1, :, s] += 1.0
    r = run(sc, vv, gg)
    leak = 0.0
    for i, s in enumerate(pos):
        d = np.abs(r[i + 1, :, :s].astype(np.float64) - r[0, :, :s].astype(np.float64))
        if d.size:
            leak = max(leak, float(d.max()))
    rms = float(np.sqrt(np.mean(r[0].astype(np.float64) ** 2)))
    print("fp32 leakage max_{t<s}|dr_t| = %.3g (rms r = %.3g)" % (leak, rms), flush=True)
    assert np.isfinite(leak)
    assert leak < 1e-3 * rms     # round-off sized, not a structural leak


def test_empty_inputs_on_every_call(sc):
    # a zero batch, channel or length dimension: every call succeeds with an empty result
    dev = "cuda:0"
    for B, C, L in ((0, 64, 16), (2, 0, 16), (2, 64, 0)):
        print("case empty B=%d C=%d L=%d" % (B, C, L), flush=True)
        f = torch.zeros((B, C, L), dtype=torch.float32, device=dev)
        t = f.transpose(1, 2).contiguous()
        W = torch.zeros((C, 64, 3), dtype=torch.float32, device=dev)
        assert sc.causal_conv(f.bfloat16(), f.bfloat16()).shape == f.shape
        assert sc.causal_conv(f.int(), f.int()).shape == f.shape
        assert all(x.shape == f.shape for x in sc.causal_conv_bwd(f, f, f))
        assert sc.causal_conv_fixed(f, f, 8, 8).shape == f.shape
        assert sc.causal_conv_blc(t, t).shape == t.shape
        assert sc.gate(f, W).shape == f.shape
        assert sc.gate_conv(f, f, W).shape == f.shape
        assert sc.gate_conv_blc(t, t, W).shape == t.shape
        k = torch.zeros((C, L), dtype=torch.float32, device=dev)
        assert sc.causal_conv_shared(f, k).shape == f.shape
    torch.cuda.synchronize()


@pytest.mark.parametrize("L,cid", [(4096, 3), (3000, 3), (3000, 4), (2056, 4), (3001, 4),
                                   (1024, 4), (777, 3), (2048, 3), (1500, 4)])
def test_many_channels_same_bits(sc, L, cid):
    # more channels than workgroups resident at once (several generations of workgroups, each
    # touching the next generation's inputs) through the M = 1024, 2048 and 4096 kernels:
    # every channel carries the bits of a call of 100 channels, in both directions, and a few
    # channels are checked on the oracle
    C = 1500
    v, g = make_inputs(WORKLOADS[cid], B=1, C=C, L=L, seed_offset=L + cid)
    dr, _ = make_inputs(WORKLOADS[cid], B=1, C=C, L=L, seed_offset=L + cid + 7)
    print("case many channels L=%d %s" % (L, "bf16" if v.dtype == np.uint16 else "f32"), flush=True)
    tv, tg, td = to_device(v), to_device(g), to_device(dr)
    r = sc.causal_conv(tv, tg)
    dv, dg = sc.causal_conv_bwd(td, tv, tg)
    bits = torch.int16 if v.dtype == np.uint16 else torch.int32
    for c0 in (0, 511, 1024, 1400):
        sl = slice(c0, c0 + 100)
        pv, pg, pd = (x[:, sl].contiguous() for x in (tv, tg, td))
        assert torch.equal(sc.causal_conv(pv, pg).view(bits), r[:, sl].view(bits)), c0
        qv, qg = sc.causal_conv_bwd(pd, pv, pg)
        assert torch.equal(qv.view(bits), dv[:, sl].view(bits)), c0
        assert torch.equal(qg.view(bits), dg[:, sl].view(bits)), c0
    torch.cuda.synchronize()
    chans = np.array([0, 511, 512, 513, 1023, 1024, C - 1])
    r_ref, S = oracle.causal_conv_f64(v[0, chans], g[0, chans])
    assert_within_bound(to_host(r)[0, chans], r_ref, S, v.dtype == np.uint16, "many channels")


def _bf16_rne(x32: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bits, nearest with ties to even (finite values)."""
    b = x32.astype(np.float32).view(np.uint32).astype(np.uint64)
    return ((b + 0x7FFF + ((b >> 16) & 1)) >> 16).astype(np.uint16)


def _near_ties_only(bf: np.ndarray, x32: np.ndarray, S: np.ndarray, what: str,
                    rel: float = 1e-5) -> float:
    """bf (bf16 bits) must be the rounding of x32, or the rounding of another value within
    rel * S_t of x32: then either x32 lies within that distance of the tie between the two
    roundings, or (outputs near zero, where a sign may flip) both lie within it of x32.
    Returns the fraction of outputs that differ from the rounding of x32."""
    rn = _bf16_rne(x32)
    diff = bf != rn
    if diff.any():
        a, b = decode(bf[diff]), decode(rn[diff])
        x, tol = x32[diff].astype(np.float64), rel * S[diff]
        tie = np.abs(x - 0.5 * (a + b)) <= tol
        near = np.maximum(np.abs(a - x), np.abs(b - x)) <= tol
        ok = tie | near
        if not ok.all():
            i = int(np.argmin(ok))
            raise AssertionError("%s: %d outputs are no rounding of a value within %g S_t "
                                 "(bf16 %r, fp32 call %r, S %r)" % (
                                     what, int((~ok).sum()), rel, float(a[i]), float(x[i]),
                                     float(S[diff][i])))
    return float(diff.mean())


@pytest.mark.parametrize("L", [4096, 3001, 2049])
def test_bf16_storage_matches_fp32_arithmetic(sc, L):
    # the bf16 call computes in fp32 and rounds once at the store: each of its outputs (and
    # gradients) is the bf16 rounding of the fp32-storage call's value on the same inputs, or
    # of a value within 1e-5 S_t of it (10x inside the fp32 bound), which a change to the
    # bf16 path's arithmetic alone may not exceed
    v, g = make_inputs(WORKLOADS[3], B=2, C=24, L=L, seed_offset=101 + L)
    print("case bf16 vs fp32 arithmetic L=%d" % L, flush=True)
    tv, tg = to_device(v), to_device(g)
    r_bf = to_host(sc.causal_conv(tv, tg))
    r_32 = to_host(sc.causal_conv(tv.float(), tg.float()))
    _, S = oracle.causal_conv_f64(v, g)
    frac = _near_ties_only(r_bf, r_32, S, "forward L=%d" % L)
    dr, _ = make_inputs(WORKLOADS[3], B=2, C=24, L=L, seed_offset=202 + L)
    td = to_device(dr)
    dv_bf, dg_bf = (to_host(x) for x in sc.causal_conv_bwd(td, tv, tg))
    dv_32, dg_32 = (to_host(x) for x in sc.causal_conv_bwd(td.float(), tv.float(), tg.float()))
    # bound scales of the gradients: the correlation sums of |dr| with |g| and with |v|
    rev = lambda a: np.ascontiguousarray(a[..., ::-1])
    _, Sv = oracle.causal_conv_f64(rev(dr), g)
    _, Sg = oracle.causal_conv_f64(rev(dr), v)
    fv = _near_ties_only(dv_bf, dv_32, rev(Sv), "dv L=%d" % L)
    fg = _near_ties_only(dg_bf, dg_32, rev(Sg), "dg L=%d" % L)
    print("bf16 vs fp32 L=%d: neighbour taken at %.2e %.2e %.2e of outputs" % (L, frac, fv, fg),
          flush=True)
