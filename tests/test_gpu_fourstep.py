"""GPU parity of the four-step (HBM-staged) path against the float64 oracle."""
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


def run(sc, v, g, **kw):
    out = sc.causal_conv(to_device(v), to_device(g), **kw)
    torch.cuda.synchronize()
    return to_host(out)


def check(sc, v, g, what, chans=None, **kw):
    r = run(sc, v, g, **kw)
    L = v.shape[-1]
    if chans is not None:
        v = v.reshape(-1, L)[chans]
        g = g.reshape(-1, L)[chans]
        r = r.reshape(-1, L)[chans]
    r_ref, S = oracle.causal_conv_f64(v, g)
    worst = assert_within_bound(r, r_ref, S, v.dtype == np.uint16, what)
    print("%s: worst err/bound = %.3g" % (what, worst), flush=True)
    return worst


@pytest.mark.parametrize("L", [2049, 3000, 4096])
def test_forced_four_step_small(sc, L):
    v, g = make_inputs(WORKLOADS[4], B=2, C=8, L=L, seed_offset=L)
    check(sc, v, g, "four-step forced L=%d" % L, path=sc.PATH_FOUR_STEP)


@pytest.mark.parametrize("L", [4097, 5000, 8192, 16384])
def test_auto_four_step(sc, L):
    v, g = make_inputs(WORKLOADS[4], B=1, C=8, L=L, seed_offset=L)
    check(sc, v, g, "four-step L=%d" % L)


def test_four_step_conv_gate_and_bf16(sc):
    v, g = make_inputs(WORKLOADS[2], B=1, C=8, L=8192, seed_offset=11)
    check(sc, v, g, "four-step conv gate f32 L=8192")
    v, g = make_inputs(WORKLOADS[3], B=1, C=8, L=8192, seed_offset=12)
    check(sc, v, g, "four-step bf16 L=8192")


def test_four_step_L65536_few_channels(sc):
    v, g = make_inputs(WORKLOADS[4], B=1, C=4)
    check(sc, v, g, "four-step L=65536")


def test_four_step_several_chunks(sc):
    # more channels than one scratch chunk holds, so the call loops over chunks
    L = 16384
    per = sc.sc_workspace_bytes(sc.KIND_F32, 1, 1, L)
    chunk = sc.sc_workspace_bytes(sc.KIND_F32, 1, 10**6, L) // per
    C = chunk + 37
    assert sc.sc_workspace_bytes(sc.KIND_F32, 1, C, L) < per * C
    v, g = make_inputs(WORKLOADS[4], B=1, C=C, L=L, seed_offset=13)
    h = chunk // 2
    chans = np.array([0, 1, h - 1, h, h + 1, chunk - 1, chunk, chunk + 1, C - 1])
    check(sc, v, g, "four-step %d channels (chunk %d)" % (C, chunk), chans=chans)


def test_four_step_two_streams_same_bits(sc):
    # a call with more channels than half a chunk alternates its parts between the caller's
    # stream and a second one; calls of at most half a chunk stay on one stream: the same
    # kernels per channel, so the same bits
    L = 16384
    per = sc.sc_workspace_bytes(sc.KIND_F32, 1, 1, L)
    chunk = sc.sc_workspace_bytes(sc.KIND_F32, 1, 10**6, L) // per
    h = chunk // 2
    C = chunk + 37
    v, g = make_inputs(WORKLOADS[4], B=1, C=C, L=L, seed_offset=16)
    print("case four-step two streams C=%d half chunk %d" % (C, h), flush=True)
    tv, tg = to_device(v), to_device(g)
    whole = sc.causal_conv(tv, tg)
    parts = [sc.causal_conv(tv[:, c0:c0 + h].contiguous(), tg[:, c0:c0 + h].contiguous())
             for c0 in range(0, C, h)]
    torch.cuda.synchronize()
    assert torch.equal(whole.view(torch.int32), torch.cat(parts, dim=1).view(torch.int32))
    # and the gradient calls, which share the launcher
    dr = to_device(make_inputs(WORKLOADS[4], B=1, C=C, L=L, seed_offset=17)[0])
    dv, dg = sc.causal_conv_bwd(dr, tv, tg)
    for c0 in range(0, C, h):
        pv, pg = sc.causal_conv_bwd(dr[:, c0:c0 + h].contiguous(), tv[:, c0:c0 + h].contiguous(),
                                    tg[:, c0:c0 + h].contiguous())
        assert torch.equal(dv[:, c0:c0 + h].view(torch.int32), pv.view(torch.int32))
        assert torch.equal(dg[:, c0:c0 + h].view(torch.int32), pg.view(torch.int32))


def test_long_full_size_sampled(sc):
    # the whole long workload (B=1, C=1536, L=65536) in one call, the launch configuration
    # the benchmark times; 64 seeded channels (always the first and the last) checked on
    # every output against the full oracle (2.1e9 multiply-adds per channel)
    w = WORKLOADS[4]
    v, g = make_inputs(w)
    rng = np.random.default_rng(np.random.SeedSequence([w.cid, 64]))
    inner = rng.choice(np.arange(1, w.C - 1), size=62, replace=False)
    chans = np.sort(np.concatenate([[0, w.C - 1], inner]))
    check(sc, v, g, "long shape sampled (64 channels)", chans=chans)


def test_caller_workspace_and_errors(sc):
    L = 8192
    v, g = make_inputs(WORKLOADS[4], B=1, C=16, L=L, seed_offset=14)
    tv, tg = to_device(v), to_device(g)
    need = sc.sc_workspace_bytes(sc.KIND_F32, 1, 16, L)
    assert need > 0
    ws = torch.empty(need, dtype=torch.uint8, device="cuda:0")
    a = sc.causal_conv(tv, tg, workspace=ws)
    b = sc.causal_conv(tv, tg)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int32), b.view(torch.int32))      # bitwise, same plan
    small = torch.empty(need - 256, dtype=torch.uint8, device="cuda:0")
    with pytest.raises(sc.SpecConvError) as ei:
        sc.causal_conv(tv, tg, workspace=small)
    assert ei.value.status == sc.SC_ERR_WORKSPACE
    # the fused path needs no workspace
    assert sc.sc_workspace_bytes(sc.KIND_F32, 8, 1024, 4096) == 0


def test_four_step_deterministic(sc):
    v, g = make_inputs(WORKLOADS[4], B=1, C=32, L=16384, seed_offset=15)
    a = run(sc, v, g)
    b = run(sc, v, g)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


def test_four_step_concurrent_callers(sc):
    # two host threads, each on a stream of its own, call the two-stream path at the same
    # time: they share the device's second stream and its events, and each call must still
    # see only its own inputs and finish before its caller's stream goes on
    import threading
    L = 16384
    per = sc.sc_workspace_bytes(sc.KIND_F32, 1, 1, L)
    chunk = sc.sc_workspace_bytes(sc.KIND_F32, 1, 10**6, L) // per
    C = chunk // 2 + 40
    dev = []
    for k in range(2):
        v, g = make_inputs(WORKLOADS[4], B=1, C=C, L=L, seed_offset=20 + k)
        dev.append((to_device(v), to_device(g)))
    ref = [sc.causal_conv(a, b) for a, b in dev]
    torch.cuda.synchronize()
    print("case four-step concurrent callers C=%d" % C, flush=True)
    outs = [[None] * 3 for _ in range(2)]
    errs = []

    def work(k):
        try:
            s = torch.cuda.Stream()
            with torch.cuda.stream(s):
                for i in range(3):
                    outs[k][i] = sc.causal_conv(*dev[k])
            s.synchronize()
        except Exception as e:  # reported on the main thread
            errs.append(e)

    threads = [threading.Thread(target=work, args=(k,)) for k in range(2)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert not errs, errs
    for k in range(2):
        for i in range(3):
            assert torch.equal(outs[k][i].view(torch.int32), ref[k].view(torch.int32)), (k, i)


@pytest.mark.parametrize("wl,L", [(4, 1 << 22), (3, (1 << 22) - 3)])
def test_four_step_longest_length_sampled(sc, wl, L):
    # the longest length the library takes (2^22, and a ragged one just below it in bf16):
    # sampled outputs, the first and last positions of each channel among them, against
    # the float64 oracle summed one output at a time
    v, g = make_inputs(WORKLOADS[wl], B=1, C=2, L=L, seed_offset=70 + wl)
    print("case four-step longest wl=%d L=%d" % (wl, L), flush=True)
    r = run(sc, v, g).reshape(2, L)
    rng = np.random.default_rng(L)
    t = np.concatenate([[0, 1, 31, 32, 33, 4095, 4096, L // 2, L - 2, L - 1],
                        rng.integers(0, L, 150)])
    ch = np.repeat(np.arange(2), t.size)
    t = np.tile(t, 2)
    r_ref, S = oracle.causal_conv_f64_at(v.reshape(2, L), g.reshape(2, L), ch, t)
    worst = assert_within_bound(r[ch, t], r_ref, S, v.dtype == np.uint16,
                                "four-step L=%d sampled" % L)
    print("four-step L=%d: worst err/bound = %.3g" % (L, worst), flush=True)
