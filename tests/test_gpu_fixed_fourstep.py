"""GPU parity of the exactly causal real-valued path above L = 4096 (sc_causal_conv_fixed_f32
through the four-step split, once per prime, and one recombining kernel) against the oracle,
bit for bit.

Lengths up to 16384 are checked at every output against the full 128-bit oracle; the
long-context shape (C = 1536, L = 65536, several chunks of channels) on seeded sampled
outputs, each summed exactly by the oracle in Python integers.  As for the fused path, no
output may move when a later input changes ("Catastrophic Token Leakage ...", abstract).
"""
import ctypes

import numpy as np
import pytest
import torch

import oracle
from tests.gpu_util import to_device, to_host
from workloads import WORKLOADS, make_inputs

pytestmark = pytest.mark.gpu
W2 = WORKLOADS[2]


@pytest.fixture(scope="module")
def sc():
    import fft_causal_long_amd as m
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return m


def run(sc, v, g, fv, fg, **kw):
    out = sc.causal_conv_fixed(to_device(v), to_device(g), fv, fg, **kw)
    torch.cuda.synchronize()
    return to_host(out)


def assert_bits(r, ref, what):
    diff = r.view(np.uint32) != ref.view(np.uint32)
    assert not diff.any(), "%s: %d of %d outputs differ; first at %s (gpu %r, ref %r)" % (
        what, int(diff.sum()), diff.size, np.argwhere(diff)[0], r[diff][0], ref[diff][0])


def check(sc, v, g, fv, fg, what):
    L = v.shape[-1]
    assert sc.sc_fixed_range_ok(float(np.abs(v).max()), float(np.abs(g).max()), fv, fg, L)
    print("case %s: shape %s fv=%d fg=%d" % (what, v.shape, fv, fg), flush=True)
    assert_bits(run(sc, v, g, fv, fg), oracle.causal_conv_fixed_f32(v, g, fv, fg), what)


@pytest.mark.parametrize("L", [4097, 5000, 8192, 8193, 12345, 16384])
def test_lengths_bit_exact(sc, L):
    v, g = make_inputs(W2, B=1, C=2, L=L, seed_offset=L)
    check(sc, v, g, 24, 24, "L=%d" % L)


@pytest.mark.parametrize("fv,fg", [(0, 0), (8, 30), (36, 36)])
def test_fraction_bits(sc, fv, fg):
    # wide fraction ranges push R past 2^64 and use all three residues
    rng = np.random.default_rng((fv + 100) * 1000 + fg)
    L = 6000
    v = rng.standard_normal((1, 2, L)).astype(np.float32)
    g = rng.standard_normal((1, 2, L)).astype(np.float32)
    if fv + fg > 60:
        v *= np.float32(2.0 ** -4)
        g *= np.float32(2.0 ** -4)
    if fv == 0:
        v *= np.float32(1000.0)
        g *= np.float32(1000.0)
    check(sc, v, g, fv, fg, "fv=%d fg=%d" % (fv, fg))


def test_near_the_exact_range(sc):
    # L * max|V| * max|G| just inside (p_A p_B p_C - 1) / 2 at L = 5000
    rng = np.random.default_rng(17)
    L = 5000
    v = (rng.uniform(-1, 1, (1, 2, L)) * 2.0 ** 37).astype(np.float32)
    g = (rng.uniform(-1, 1, (1, 2, L)) * 2.0 ** 37).astype(np.float32)
    v[0, :, :64] = np.float32(2.0 ** 37)
    g[0, :, :64] = np.float32(2.0 ** 37)
    check(sc, v, g, 0, 0, "large encodings L=5000")


def test_forced_path_and_workspace(sc):
    L = 6000
    v, g = make_inputs(W2, B=2, C=3, L=L, seed_offset=23)
    a = run(sc, v, g, 20, 22)
    # the four-step path forced through sc_causal_conv_ex gives the same bits
    h = sc.lib()
    tv, tg = to_device(v), to_device(g)
    out = torch.empty_like(tv)
    opt = sc.sc_options(sc.PATH_FOUR_STEP, -1, 20, 22)
    st = h.sc_causal_conv_ex(sc.KIND_FIXED_F32, tv.data_ptr(), tg.data_ptr(), out.data_ptr(),
                             2, 3, L, ctypes.byref(opt), None, 0,
                             torch.cuda.current_stream().cuda_stream)
    assert st == sc.SC_OK, sc.sc_status_string(st)
    torch.cuda.synchronize()
    assert np.array_equal(to_host(out).view(np.uint32), a.view(np.uint32))
    # a caller workspace of exactly the reported size
    need = sc.sc_workspace_bytes(sc.KIND_FIXED_F32, 2, 3, L)
    assert need == 6 * 40 * 8192
    ws = torch.empty(need, dtype=torch.uint8, device="cuda:0")
    b = run(sc, v, g, 20, 22, workspace=ws)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
    assert_bits(a, oracle.causal_conv_fixed_f32(v, g, 20, 22), "forced/workspace")


def test_exact_causality(sc):
    L = 8192
    v, g = make_inputs(W2, B=1, C=2, L=L, seed_offset=29)
    base = run(sc, v, g, 24, 24)
    for s in (1, 4095, 4096, 6000, L - 1):
        v2, g2 = v.copy(), g.copy()
        v2[..., s] += np.float32(0.5)
        g2[..., s] -= np.float32(0.25)
        r2 = run(sc, v2, g2, 24, 24)
        assert np.array_equal(r2[..., :s].view(np.uint32), base[..., :s].view(np.uint32)), s
        assert not np.array_equal(r2[..., s], base[..., s])


def test_long_context_shape_sampled(sc):
    # C = 1536 channels of L = 65536 (several chunks): 4 seeded outputs (and the last) on
    # each of 48 seeded channels, always including the first and the last channel
    w = WORKLOADS[4]
    v, g = make_inputs(w, seed_offset=37)
    assert sc.sc_fixed_range_ok(float(np.abs(v).max()), float(np.abs(g).max()), 24, 24, w.L)
    print("case fixed long shape: %s" % (v.shape,), flush=True)
    r = run(sc, v, g, 24, 24).reshape(-1, w.L)
    rng = np.random.default_rng(np.random.SeedSequence([4, 37]))
    chans = np.concatenate([[0, w.C - 1], rng.choice(np.arange(1, w.C - 1), 46, replace=False)])
    ch = np.repeat(chans, 5)
    t = rng.integers(0, w.L, size=ch.size)
    t[::5] = w.L - 1
    want = oracle.causal_conv_fixed_f32_at(v.reshape(-1, w.L), g.reshape(-1, w.L), 24, 24, ch, t)
    assert_bits(r[ch, t], want, "long shape sampled")


def test_parts_agree_across_partitions(sc):
    # The long-context shape in one call (chunks run as halves on two streams) and as three
    # calls on slices of its channels, whose chunks and halves fall elsewhere: every output
    # must agree bit for bit.
    w = WORKLOADS[4]
    v, g = make_inputs(w, seed_offset=47)
    assert sc.sc_fixed_range_ok(float(np.abs(v).max()), float(np.abs(g).max()), 24, 24, w.L)
    print("case fixed long shape partitions: %s" % (v.shape,), flush=True)
    tv, tg = to_device(v), to_device(g)
    whole = sc.causal_conv_fixed(tv, tg, 24, 24)
    for c0, c1 in [(0, 100), (100, 433), (433, w.C)]:
        part = sc.causal_conv_fixed(tv[:, c0:c1].contiguous(), tg[:, c0:c1].contiguous(), 24, 24)
        torch.cuda.synchronize()
        assert torch.equal(part.view(torch.int32), whole[:, c0:c1].view(torch.int32)), (c0, c1)


def test_graph_capture_after_prepare(sc):
    L = 12288
    v, g = make_inputs(W2, B=1, C=3, L=L, seed_offset=41)
    assert sc.sc_prepare(sc.KIND_FIXED_F32, L) == sc.SC_OK
    tv, tg = to_device(v), to_device(g)
    need = sc.sc_workspace_bytes(sc.KIND_FIXED_F32, 1, 3, L)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda:0")
    eager = sc.causal_conv_fixed(tv, tg, 24, 24, workspace=ws)
    torch.cuda.synchronize()
    out = torch.empty_like(tv)
    s = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=s):
        sc.causal_conv_fixed(tv, tg, 24, 24, out, workspace=ws)
    for _ in range(3):
        out.fill_(0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int32), eager.view(torch.int32))


def test_token_major(sc):
    # (B, L, C) inputs through the staged token-major call, whose inner call takes the
    # four-step split: bitwise the channel-major result
    B, L, C = 2, 5000, 6
    v, g = make_inputs(W2, B=B, C=C, L=L, seed_offset=43)
    a = run(sc, v, g, 24, 24)
    vt = to_device(np.ascontiguousarray(v.transpose(0, 2, 1)))
    gt = to_device(np.ascontiguousarray(g.transpose(0, 2, 1)))
    rt = torch.empty_like(vt)
    opt = sc.sc_options(sc.PATH_AUTO, -1, 24, 24)
    print("case fixed token-major L=%d" % L, flush=True)
    st = sc.sc_causal_conv_blc_ex(sc.KIND_FIXED_F32, vt.data_ptr(), gt.data_ptr(), rt.data_ptr(),
                                  B, L, C, ctypes.byref(opt), None, 0,
                                  torch.cuda.current_stream().cuda_stream)
    assert st == sc.SC_OK, sc.sc_status_string(st)
    torch.cuda.synchronize()
    got = np.ascontiguousarray(to_host(rt).transpose(0, 2, 1))
    assert np.array_equal(got.view(np.uint32), a.view(np.uint32))
