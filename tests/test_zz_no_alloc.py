"""The allocation-free entry point sc_causal_conv_noalloc against the entry point it
varies (sc_causal_conv_ex with a caller workspace), through the C ABI: the same bits on
the four-step path (whose scratch is the library's static device array), on two calls in a
row, the second with a smaller input, and on the fused path.  Its tables come from
sc_prepare, so the call itself allocates nothing."""
import numpy as np
import pytest
import torch

from tests.gpu_util import to_device
from workloads import WORKLOADS, make_inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def sc():
    import fft_causal_long_amd as m
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return m


def bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


def reference(sc, kind, vd, gd, B, C, L):
    need = sc.sc_workspace_bytes(kind, B, C, L)
    ws = torch.empty(max(need, 256), dtype=torch.uint8, device="cuda:0")
    out = torch.empty_like(vd)
    st = sc.lib().sc_causal_conv_ex(kind, vd.data_ptr(), gd.data_ptr(), out.data_ptr(), B, C, L,
                                    None, ws.data_ptr() if need else None, need,
                                    torch.cuda.current_stream().cuda_stream)
    assert st == sc.SC_OK, sc.sc_status_string(st)
    return out


def noalloc(sc, kind, vd, gd, out, B, C, L):
    return sc.lib().sc_causal_conv_noalloc(kind, vd.data_ptr(), gd.data_ptr(), out.data_ptr(),
                                           B, C, L, torch.cuda.current_stream().cuda_stream)


@pytest.mark.parametrize("w_id,kind", [(4, 0), (3, 1)])
def test_two_calls_in_a_row_match_the_workspace_call(sc, w_id, kind):
    w = WORKLOADS[w_id]
    L = 65536
    # 64 MiB of static scratch holds 42 channels at L = 65536: the first call runs in three
    # parts, the second (smaller) in one
    shapes = [(2, 50, L), (1, 7, 20000)]
    for L_ in sorted({s[2] for s in shapes}):
        assert sc.sc_prepare(kind, L_) == sc.SC_OK
    outs = []
    for i, (B, C, L_) in enumerate(shapes):
        v, g = make_inputs(w, B=B, C=C, L=L_, seed_offset=90 + i)
        vd, gd = to_device(v), to_device(g)
        out = torch.full_like(vd, 3.0)
        print("case noalloc kind=%d B=%d C=%d L=%d" % (kind, B, C, L_), flush=True)
        assert noalloc(sc, kind, vd, gd, out, B, C, L_) == sc.SC_OK
        outs.append((out, vd, gd, B, C, L_))
    torch.cuda.synchronize()
    for out, vd, gd, B, C, L_ in outs:
        ref = reference(sc, kind, vd, gd, B, C, L_)
        torch.cuda.synchronize()
        assert torch.equal(bits(out), bits(ref)), (B, C, L_)


def test_fused_and_exact_paths(sc):
    for w_id, kind, L in ((3, 1, 4096), (5, 2, 4096), (2, 0, 1000)):
        w = WORKLOADS[w_id]
        v, g = make_inputs(w, B=2, C=16, L=L, seed_offset=95)
        vd, gd = to_device(v), to_device(g)
        assert sc.sc_prepare(kind, L) == sc.SC_OK
        out = torch.empty_like(vd)
        print("case noalloc fused kind=%d L=%d" % (kind, L), flush=True)
        assert noalloc(sc, kind, vd, gd, out, 2, 16, L) == sc.SC_OK
        ref = reference(sc, kind, vd, gd, 2, 16, L)
        torch.cuda.synchronize()
        assert torch.equal(bits(out), bits(ref)), (w_id, kind)


def test_refusals(sc):
    v = torch.zeros(1 << 22, dtype=torch.float32, device="cuda:0")
    g, r = torch.zeros_like(v), torch.zeros_like(v)
    s = torch.cuda.current_stream().cuda_stream
    f = sc.lib().sc_causal_conv_noalloc
    # one channel of this length needs more than the static scratch
    assert f(0, v.data_ptr(), g.data_ptr(), r.data_ptr(), 1, 1, (1 << 21) + 1, s) == \
        sc.SC_ERR_UNSUPPORTED
    # the fixed-point kind is not offered
    assert f(3, v.data_ptr(), g.data_ptr(), r.data_ptr(), 1, 1, 64, s) == \
        sc.SC_ERR_INVALID_ARGUMENT
    torch.cuda.synchronize()
