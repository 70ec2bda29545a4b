"""The library under HIP graph capture: the fused call, the token-major call (caller
workspace), a four-step call and the gradient calls are captured in a torch CUDA graph on a side stream, the graph is replayed several
times with the program's own eager work in between, and every replay must equal the eager
result bit for bit.  The library allocates nothing on these paths, so capture is valid."""
import numpy as np
import pytest
import torch

from tests.gpu_util import to_device, to_host
from workloads import WORKLOADS, make_inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def sc():
    import fft_causal_long_amd as m
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return m


def replay_check(graph, out, ref, refresh):
    for i in range(3):
        out.zero_()
        refresh(i)                       # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16) if out.dtype == torch.bfloat16 else out,
                           ref.view(torch.int16) if ref.dtype == torch.bfloat16 else ref), i


def test_fused_call_in_a_graph(sc):
    v, g = make_inputs(WORKLOADS[3], B=2, C=64, L=4096, seed_offset=61)
    vd, gd = to_device(v), to_device(g)
    ref = sc.causal_conv(vd, gd)
    out = torch.empty_like(ref)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    print("case graph fused", flush=True)
    with torch.cuda.stream(side):
        sc.causal_conv(vd, gd, out=out)          # warm-up on the capture stream
        torch.cuda.synchronize()
        with torch.cuda.graph(graph, stream=side):
            sc.causal_conv(vd, gd, out=out)
    torch.cuda.synchronize()
    replay_check(graph, out, ref, lambda i: torch.mul(vd, 1, out=torch.empty_like(vd)))


def test_token_major_call_in_a_graph(sc):
    B, L, C = 2, 1000, 130
    v, g = make_inputs(WORKLOADS[2], B=B, C=C, L=L, seed_offset=62)
    vt = to_device(np.ascontiguousarray(np.swapaxes(v, 1, 2)))
    gt = to_device(np.ascontiguousarray(np.swapaxes(g, 1, 2)))
    ws = torch.empty(sc.sc_blc_workspace_bytes(sc.KIND_F32, B, L, C), dtype=torch.uint8,
                     device="cuda:0")
    ref = sc.causal_conv_blc(vt, gt, workspace=ws)
    out = torch.empty_like(ref)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    print("case graph token-major", flush=True)
    with torch.cuda.stream(side):
        sc.causal_conv_blc(vt, gt, out=out, workspace=ws)
        torch.cuda.synchronize()
        with torch.cuda.graph(graph, stream=side):
            sc.causal_conv_blc(vt, gt, out=out, workspace=ws)
    torch.cuda.synchronize()
    # eager work that reuses the workspace between replays
    replay_check(graph, out, ref,
                 lambda i: sc.causal_conv_blc(vt, gt, out=torch.empty_like(vt), workspace=ws))


def test_four_step_call_in_a_graph(sc):
    # eagerly, this many channels alternate between the caller's stream and a second one;
    # under capture the call must stay on the capturing stream (caller workspace, tables made
    # by the warm-up call), and every replay must give the eager bits
    L = 16384
    per = sc.sc_workspace_bytes(sc.KIND_F32, 1, 1, L)
    chunk = sc.sc_workspace_bytes(sc.KIND_F32, 1, 10**6, L) // per
    C = chunk // 2 + 44
    v, g = make_inputs(WORKLOADS[4], B=1, C=C, L=L, seed_offset=63)
    vd, gd = to_device(v), to_device(g)
    ws = torch.empty(sc.sc_workspace_bytes(sc.KIND_F32, 1, C, L), dtype=torch.uint8,
                     device="cuda:0")
    ref = sc.causal_conv(vd, gd, workspace=ws)
    out = torch.empty_like(ref)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    print("case graph four-step C=%d L=%d" % (C, L), flush=True)
    with torch.cuda.stream(side):
        sc.causal_conv(vd, gd, out=out, workspace=ws)
        torch.cuda.synchronize()
        with torch.cuda.graph(graph, stream=side):
            sc.causal_conv(vd, gd, out=out, workspace=ws)
    torch.cuda.synchronize()
    # eager two-stream calls that reuse the workspace between replays
    replay_check(graph, out, ref,
                 lambda i: sc.causal_conv(vd, gd, out=torch.empty_like(vd), workspace=ws))


def test_gradient_and_empty_batch_calls_in_a_graph(sc):
    # the gradient call (fused path) and the shared-filter gradients of an empty batch (whose
    # dk is cleared by a fill kernel, not a memset) captured together; every replay gives the
    # eager dv, dg bit for bit and a zero dk
    v, g = make_inputs(WORKLOADS[3], B=2, C=64, L=4096, seed_offset=64)
    dr = make_inputs(WORKLOADS[3], B=2, C=64, L=4096, seed_offset=65)[0]
    vd, gd, drd = to_device(v), to_device(g), to_device(dr)
    rdv, rdg = sc.causal_conv_bwd(drd, vd, gd)
    dv, dg = torch.empty_like(rdv), torch.empty_like(rdg)
    e = torch.empty((0, 3, 333), dtype=torch.bfloat16, device="cuda:0")
    k = torch.ones((3, 333), dtype=torch.bfloat16, device="cuda:0")
    dk = torch.full((3, 333), 7.0, dtype=torch.bfloat16, device="cuda:0")
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    print("case graph gradients + empty batch", flush=True)
    with torch.cuda.stream(side):
        sc.causal_conv_bwd(drd, vd, gd, dv=dv, dg=dg)
        sc.causal_conv_shared_bwd(e, e, k, dk=dk)
        torch.cuda.synchronize()
        with torch.cuda.graph(graph, stream=side):
            sc.causal_conv_bwd(drd, vd, gd, dv=dv, dg=dg)
            sc.causal_conv_shared_bwd(e, e, k, dk=dk)
    torch.cuda.synchronize()
    for i in range(3):
        dv.zero_()
        dg.zero_()
        dk.fill_(7.0)
        torch.mul(vd, 1, out=torch.empty_like(vd))       # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(dv.view(torch.int16), rdv.view(torch.int16)), i
        assert torch.equal(dg.view(torch.int16), rdg.view(torch.int16)), i
        assert int(torch.count_nonzero(dk)) == 0, i


def test_four_step_call_of_several_parts_in_a_graph(sc):
    # under capture the four-step path stays on the capturing stream; with more channels than
    # one chunk its parts run one after the other and reuse the start of the workspace, which
    # is sized exactly (no slack past what the call needs): every replay gives the eager bits
    L = 16384
    per = sc.sc_workspace_bytes(sc.KIND_F32, 1, 1, L)
    chunk = sc.sc_workspace_bytes(sc.KIND_F32, 1, 10**6, L) // per
    C = chunk + 44
    v, g = make_inputs(WORKLOADS[4], B=1, C=C, L=L, seed_offset=66)
    vd, gd = to_device(v), to_device(g)
    need = sc.sc_workspace_bytes(sc.KIND_F32, 1, C, L)
    assert need == chunk * per
    ws = torch.empty(need, dtype=torch.uint8, device="cuda:0")
    ref = sc.causal_conv(vd, gd, workspace=ws)
    out = torch.empty_like(ref)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    print("case graph four-step parts C=%d chunk=%d L=%d" % (C, chunk, L), flush=True)
    with torch.cuda.stream(side):
        sc.causal_conv(vd, gd, out=out, workspace=ws)
        torch.cuda.synchronize()
        with torch.cuda.graph(graph, stream=side):
            sc.causal_conv(vd, gd, out=out, workspace=ws)
    torch.cuda.synchronize()
    replay_check(graph, out, ref,
                 lambda i: sc.causal_conv(vd, gd, out=torch.empty_like(vd), workspace=ws))


def test_capture_needing_a_new_table_is_refused_until_prepared(sc):
    # the four-step tables for M = 2^21 are built by no other test: captured before
    # sc_prepare, the call must refuse (nothing enqueued, the capture stays valid); after
    # sc_prepare the same capture succeeds and replays give the eager bits
    L = (1 << 20) + 3
    v, g = make_inputs(WORKLOADS[4], B=1, C=2, L=L, seed_offset=67)
    vd, gd = to_device(v), to_device(g)
    need = sc.sc_workspace_bytes(sc.KIND_F32, 1, 2, L)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda:0")
    out = torch.empty_like(vd)
    fn = sc.lib().sc_causal_conv_f32_ws
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    torch.cuda.synchronize()
    print("case graph refused before sc_prepare L=%d" % L, flush=True)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            st = fn(vd.data_ptr(), gd.data_ptr(), out.data_ptr(), 1, 2, L, ws.data_ptr(), need,
                    side.cuda_stream)
            torch.mul(vd, 1, out=out)          # keeps the captured graph non-empty
    torch.cuda.synchronize()
    assert st == sc.SC_ERR_UNSUPPORTED
    assert sc.sc_prepare(sc.KIND_F32, L) == sc.SC_OK
    ref = sc.causal_conv(vd, gd, workspace=ws)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            st = fn(vd.data_ptr(), gd.data_ptr(), out.data_ptr(), 1, 2, L, ws.data_ptr(), need,
                    side.cuda_stream)
    torch.cuda.synchronize()
    assert st == sc.SC_OK
    replay_check(graph, out, ref, lambda i: torch.mul(vd, 1, out=torch.empty_like(vd)))
