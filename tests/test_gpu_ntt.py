"""GPU parity of the exact NTT path against the int64 oracle: bit for bit.

The oracle's exact sum is lifted to the symmetric residue range mod p = 998244353; when
|sum| <= (p-1)/2 (the workloads here) that is the integer itself.  Leakage: with the
original and perturbed rows in one launch, outputs t < s must be bitwise unchanged when
v_s changes ("Catastrophic Token Leakage ...", abstract: integer transforms cannot leak).
"""
import numpy as np
import pytest
import torch

import oracle
from tests.gpu_util import to_device, to_host
from workloads import WORKLOADS, make_inputs, perturbation_positions

pytestmark = pytest.mark.gpu
P = oracle.P_NTT


@pytest.fixture(scope="module")
def sc():
    import fft_causal_long_amd as m
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return m


def run(sc, v, g, **kw):
    out = sc.causal_conv(to_device(v), to_device(g), **kw)
    torch.cuda.synchronize()
    return to_host(out)


def test_exact_medium_full_bit_exact(sc):
    w = WORKLOADS[5]
    v, g = make_inputs(w)
    assert sc.sc_ntt_range_ok(127, 127, w.L)
    r = run(sc, v, g)
    ref = oracle.causal_conv_i64(v, g)
    assert np.abs(ref).max() <= (P - 1) // 2
    assert r.dtype == np.int32
    mism = np.count_nonzero(r.astype(np.int64) != ref)
    assert mism == 0, "%d mismatches" % mism


@pytest.mark.parametrize("L", [1, 2, 3, 17, 33, 64, 65, 100, 255, 256, 257, 1000, 1024, 2047,
                               2048, 3000, 4095, 4096])
def test_length_sweep_bit_exact(sc, L):
    v, g = make_inputs(WORKLOADS[5], B=3, C=5, L=L, seed_offset=L)
    r = run(sc, v, g)
    assert np.array_equal(r.astype(np.int64), oracle.causal_conv_i64(v, g))


def test_wraps_mod_p_beyond_the_precondition(sc):
    # |sums| far above (p-1)/2: the defined result is the lifted residue
    rng = np.random.default_rng(41)
    L = 1024
    v = rng.integers(-(2**20), 2**20, size=(4, 7, L), dtype=np.int32)
    g = rng.integers(-(2**20), 2**20, size=(4, 7, L), dtype=np.int32)
    assert not sc.sc_ntt_range_ok(2**20, 2**20, L)
    exact = oracle.causal_conv_i64(v, g)             # |.| < 2^50: exact in int64
    assert np.abs(exact).max() > P
    r = run(sc, v, g)
    assert np.array_equal(r.astype(np.int64), oracle.lift_mod_p(exact))


def test_full_range_int32_inputs(sc):
    rng = np.random.default_rng(42)
    L = 40
    v = rng.integers(-(2**31), 2**31, size=(2, 3, L), dtype=np.int64).astype(np.int32)
    g = rng.integers(-(2**31), 2**31, size=(2, 3, L), dtype=np.int64).astype(np.int32)
    v[0, 0, :3] = [-(2**31), 2**31 - 1, 0]
    r = run(sc, v, g)
    for b in range(2):
        for c in range(3):
            for t in range(L):
                s = sum(int(v[b, c, j]) * int(g[b, c, t - j]) for j in range(t + 1)) % P
                s = s - P if s > (P - 1) // 2 else s
                assert int(r[b, c, t]) == s, (b, c, t)


def test_ntt_leakage_is_exactly_zero(sc):
    w = WORKLOADS[5]
    L = w.L
    v, g = make_inputs(w, B=1, C=32)
    pos = perturbation_positions(w.cid, L)
    rng = np.random.default_rng(43)
    vv = np.concatenate([v] + [v.copy() for _ in pos], axis=0)
    gg = np.concatenate([g] * (len(pos) + 1), axis=0)
    for i, s in enumerate(pos):
        new = rng.integers(-127, 128, size=v.shape[1], dtype=np.int32)
        new = np.where(new == v[0, :, s], new + 1 if s % 2 else new - 1, new)
        vv[i + 1, :, s] = np.clip(new, -127, 127)
    r = run(sc, vv, gg)
    leak = 0
    changed = 0
    for i, s in enumerate(pos):
        leak = max(leak, int(np.abs(r[i + 1, :, :s].astype(np.int64) - r[0, :, :s]).max(initial=0)))
        changed += int(np.count_nonzero(r[i + 1, :, s] != r[0, :, s]))
    print("NTT leakage max_{t<s}|dr_t| = %d over %d positions" % (leak, len(pos)), flush=True)
    assert leak == 0
    assert changed > 0          # the perturbation itself is visible at t = s
    ref = oracle.causal_conv_i64(vv, gg)
    assert np.array_equal(r.astype(np.int64), ref)


def test_deterministic(sc):
    v, g = make_inputs(WORKLOADS[5], B=1, C=64)
    a = run(sc, v, g)
    b = run(sc, v, g)
    assert np.array_equal(a, b)
