"""GPU parity of the exact NTT path with its transform stages as int8 matrix products
(SC_PATH_NTT_MFMA, "Catastrophic Token Leakage ...", abstract: the integer FFT built from
standard integer matrix multiplications) against the int64 oracle, bit for bit, and
against the butterfly kernel's bits."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
from tests.gpu_util import to_device, to_host
from workloads import WORKLOADS, make_grad, make_inputs, perturbation_positions

pytestmark = pytest.mark.gpu
P = oracle.P_NTT


@pytest.fixture(scope="module")
def sc():
    import fft_causal_long_amd as m
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return m


def run(sc, v, g, path):
    out = sc.causal_conv(to_device(v), to_device(g), path=path)
    torch.cuda.synchronize()
    return to_host(out)


def test_exact_medium_full_bit_exact(sc):
    w = WORKLOADS[5]
    v, g = make_inputs(w)
    print("case ntt-mfma exact medium full", flush=True)
    r = run(sc, v, g, sc.PATH_NTT_MFMA)
    ref = oracle.causal_conv_i64(v, g)
    assert np.abs(ref).max() <= (P - 1) // 2
    mism = np.count_nonzero(r.astype(np.int64) != ref)
    assert mism == 0, "%d mismatches" % mism
    assert np.array_equal(r, run(sc, v, g, sc.PATH_FUSED))


@pytest.mark.parametrize("L", [1, 2, 3, 17, 33, 63, 64, 65, 100, 128, 255, 256, 257, 511, 512,
                               1000, 1024, 2047, 2048, 2049, 3000, 4095, 4096])
def test_length_sweep_bit_exact(sc, L):
    v, g = make_inputs(WORKLOADS[5], B=3, C=5, L=L, seed_offset=L + 500)
    print("case ntt-mfma L=%d" % L, flush=True)
    r = run(sc, v, g, sc.PATH_NTT_MFMA)
    assert np.array_equal(r.astype(np.int64), oracle.causal_conv_i64(v, g))


def test_wraps_mod_p_and_full_range_inputs(sc):
    # sums far beyond (p-1)/2 and inputs over the whole int32 range: the lifted residue,
    # the same bits as the butterfly kernel
    rng = np.random.default_rng(51)
    L = 1024
    v = rng.integers(-(2**20), 2**20, size=(4, 7, L), dtype=np.int32)
    g = rng.integers(-(2**20), 2**20, size=(4, 7, L), dtype=np.int32)
    exact = oracle.causal_conv_i64(v, g)
    assert np.abs(exact).max() > P
    r = run(sc, v, g, sc.PATH_NTT_MFMA)
    assert np.array_equal(r.astype(np.int64), oracle.lift_mod_p(exact))
    L = 300
    v = rng.integers(-(2**31), 2**31, size=(2, 3, L), dtype=np.int64).astype(np.int32)
    g = rng.integers(-(2**31), 2**31, size=(2, 3, L), dtype=np.int64).astype(np.int32)
    v[0, 0, :3] = [-(2**31), 2**31 - 1, 0]
    g[1, 2, :2] = [2**31 - 1, -(2**31)]
    r = run(sc, v, g, sc.PATH_NTT_MFMA)
    vr, gr = np.mod(v.astype(np.int64), P), np.mod(g.astype(np.int64), P)
    for b in range(2):
        for c in range(3):
            for t in range(0, L, 7):
                s = int(np.sum((vr[b, c, :t + 1] * gr[b, c, t::-1][:t + 1]) % P) % P)
                s = s - P if s > (P - 1) // 2 else s
                assert int(r[b, c, t]) == s, (b, c, t)
    assert np.array_equal(r, run(sc, v, g, sc.PATH_FUSED))


def test_gradients_bit_exact(sc):
    w = WORKLOADS[5]
    v, g = make_inputs(w, B=2, C=16, L=4096, seed_offset=52)
    dr = make_grad(w, B=2, C=16, L=4096, seed_offset=52)
    dv, dg = sc.causal_conv_bwd(to_device(dr), to_device(v), to_device(g),
                                path=sc.PATH_NTT_MFMA)
    torch.cuda.synchronize()
    rdv, rdg = oracle.causal_conv_bwd_i64(dr, v, g)
    assert np.array_equal(to_host(dv).astype(np.int64), rdv)
    assert np.array_equal(to_host(dg).astype(np.int64), rdg)


def test_leakage_is_exactly_zero(sc):
    w = WORKLOADS[5]
    L = w.L
    v, g = make_inputs(w, B=1, C=16, seed_offset=53)
    pos = perturbation_positions(w.cid, L)
    rng = np.random.default_rng(54)
    vv = np.concatenate([v] + [v.copy() for _ in pos], axis=0)
    gg = np.concatenate([g] * (len(pos) + 1), axis=0)
    for i, s in enumerate(pos):
        vv[i + 1, :, s] = np.where(v[0, :, s] >= 0, v[0, :, s] - 100, v[0, :, s] + 100)
    r = run(sc, vv, gg, sc.PATH_NTT_MFMA)
    for i, s in enumerate(pos):
        assert np.array_equal(r[i + 1, :, :s], r[0, :, :s]), s
        assert np.count_nonzero(r[i + 1, :, s] != r[0, :, s]) > 0
    assert np.array_equal(r.astype(np.int64), oracle.causal_conv_i64(vv, gg))


def test_option_refused_for_other_kinds_and_lengths(sc):
    h = sc.lib()
    a = torch.zeros(8192, dtype=torch.float32, device="cuda:0")
    b, c = torch.zeros_like(a), torch.zeros_like(a)
    opt = sc.sc_options(sc.PATH_NTT_MFMA, -1)
    s = torch.cuda.current_stream().cuda_stream
    for kind, L in ((sc.KIND_F32, 64), (sc.KIND_BF16, 64), (sc.KIND_NTT_I32, 4097)):
        st = h.sc_causal_conv_ex(kind, a.data_ptr(), b.data_ptr(), c.data_ptr(), 1, 1, L,
                                 ctypes.byref(opt), None, 0, s)
        assert st == sc.SC_ERR_UNSUPPORTED, (kind, L)
