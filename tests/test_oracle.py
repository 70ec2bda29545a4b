"""Pins for the CPU oracle (CPU only).

The oracle is checked against things other than itself: hand-worked examples
(tests/golden/hand_cases.txt), closed forms, library routines (numpy.convolve,
numpy.fft), brute-force recipes, invariants (causality, commutativity, bilinearity),
and number-theoretic facts about the modulus.  Each check is chosen so that a dropped
term, a wrong sign or index, or a swapped operand in the oracle fails at least one.
"""
import os

import numpy as np
import pytest

import oracle
from oracle import (P_NTT, ROOT_NTT, causal_conv_f64, causal_conv_f64_at, causal_conv_i64,
                    circular_conv_dft, circular_conv_ntt, lift_mod_p)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_cases.txt")


def _golden():
    cases = []
    with open(GOLDEN) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            kind, name, v, g, out = [x.strip() for x in line.split("|")]
            cases.append((kind, name, [int(x) for x in v.split()],
                          [int(x) for x in g.split()], [int(x) for x in out.split()]))
    assert len(cases) >= 7
    return cases


@pytest.mark.parametrize("case", [c for c in _golden() if c[0] == "causal"], ids=lambda c: c[1])
def test_golden_causal(case):
    _, _, v, g, expect = case
    r64, S = causal_conv_f64(np.array(v, np.float64), np.array(g, np.float64))
    assert r64.tolist() == [float(x) for x in expect]
    ri = causal_conv_i64(np.array(v), np.array(g))
    assert ri.tolist() == expect
    assert np.all(S >= np.abs(r64))


@pytest.mark.parametrize("case", [c for c in _golden() if c[0].startswith("circ:")],
                         ids=lambda c: c[1])
def test_golden_circular(case):
    kind, _, v, g, expect = case
    n = int(kind.split(":")[1])
    d = circular_conv_dft(np.array(v, np.float64), np.array(g, np.float64), n)
    np.testing.assert_allclose(d, expect, atol=1e-12)
    t = lift_mod_p(circular_conv_ntt(np.array(v), np.array(g), n)) if (P_NTT - 1) % n == 0 else None
    if t is not None:
        assert t.tolist() == expect


def test_unpadded_wraps_future_into_past():
    # The negative control (FourierQK explainer, problem statement: periodic DFT
    # boundaries leak the future into the past): without padding, the circular result
    # differs from the causal one at t = 0 and uses v_{L-1}.
    v = np.array([1.0, 2.0])
    g = np.array([3.0, 4.0])
    r, _ = causal_conv_f64(v, g)
    c = circular_conv_dft(v, g, 2)
    assert r[0] == 3.0 and abs(c[0] - 11.0) < 1e-12
    rng = np.random.default_rng(5)
    L = 16
    v = rng.standard_normal(L)
    g = rng.standard_normal(L)
    r, _ = causal_conv_f64(v, g)
    c = circular_conv_dft(v, g, L)
    assert np.max(np.abs(c[: L - 1] - r[: L - 1])) > 1e-3
    # the last output has no future terms to wrap
    assert abs(c[L - 1] - r[L - 1]) < 1e-10


def test_closed_forms():
    L = 40
    rng = np.random.default_rng(1)
    v = rng.standard_normal(L)
    # g = delta_0  ->  r = v
    d0 = np.zeros(L)
    d0[0] = 1.0
    r, _ = causal_conv_f64(v, d0)
    assert np.array_equal(r, v)
    # g = delta_k  ->  r_t = v_{t-k}
    for k in (1, 7, 39):
        dk = np.zeros(L)
        dk[k] = 1.0
        r, _ = causal_conv_f64(v, dk)
        expect = np.concatenate([np.zeros(k), v[: L - k]])
        assert np.array_equal(r, expect)
    # g = 1  ->  running sum of v
    r, _ = causal_conv_f64(v, np.ones(L))
    np.testing.assert_allclose(r, np.cumsum(v), rtol=0, atol=1e-12)
    # v = g = 1  ->  t + 1
    r, S = causal_conv_f64(np.ones(L), np.ones(L))
    assert np.array_equal(r, np.arange(1, L + 1, dtype=np.float64))
    assert np.array_equal(S, r)
    # geometric: v_t = a^t, g_t = b^t  ->  (a^{t+1} - b^{t+1}) / (a - b)
    a, b = 0.9, -0.5
    t = np.arange(L, dtype=np.float64)
    r, _ = causal_conv_f64(a ** t, b ** t)
    np.testing.assert_allclose(r, (a ** (t + 1) - b ** (t + 1)) / (a - b), rtol=1e-13, atol=1e-15)


def test_asymmetric_roles():
    # v and g enter as v_j g_{t-j}; a swapped index (v_{t-j} g_j) is the same sum, but a
    # dropped reversal (v_j g_j) or an off-by-one (g_{t-j+1}) is not.
    v = np.array([1.0, 0.0, 0.0, 0.0])
    g = np.array([0.0, 1.0, 2.0, 3.0])
    r, _ = causal_conv_f64(v, g)
    assert r.tolist() == [0.0, 1.0, 2.0, 3.0]
    r, _ = causal_conv_f64(g, v)
    assert r.tolist() == [0.0, 1.0, 2.0, 3.0]
    v = np.array([0.0, 1.0, 0.0, 0.0])
    r, _ = causal_conv_f64(v, g)
    assert r.tolist() == [0.0, 0.0, 1.0, 2.0]


@pytest.mark.parametrize("L", [1, 2, 3, 17, 64, 255])
def test_matches_numpy_convolve(L):
    rng = np.random.default_rng(L)
    v = rng.standard_normal((3, L))
    g = rng.standard_normal((3, L))
    r, S = causal_conv_f64(v, g)
    for c in range(3):
        ref = np.convolve(v[c], g[c])[:L]
        sref = np.convolve(np.abs(v[c]), np.abs(g[c]))[:L]
        np.testing.assert_allclose(r[c], ref, rtol=0, atol=1e-13 * max(1.0, sref.max()))
        np.testing.assert_allclose(S[c], sref, rtol=1e-13)
        assert np.all(S[c] >= np.abs(r[c]) - 1e-12)
    vi = rng.integers(-127, 128, size=(3, L))
    gi = rng.integers(-127, 128, size=(3, L))
    ri = causal_conv_i64(vi, gi)
    for c in range(3):
        assert np.array_equal(ri[c], np.convolve(vi[c], gi[c])[:L])


def test_commutative_and_bilinear_exact():
    rng = np.random.default_rng(9)
    L = 200
    a, b, c = (rng.integers(-1000, 1000, size=(2, L)) for _ in range(3))
    ab = causal_conv_i64(a, b)
    assert np.array_equal(ab, causal_conv_i64(b, a))
    assert np.array_equal(causal_conv_i64(a + c, b), ab + causal_conv_i64(c, b))
    assert np.array_equal(causal_conv_i64(3 * a, b), 3 * ab)


@pytest.mark.parametrize("L", [1, 2, 5, 16, 33, 64])
def test_pad_2L_dft_recipe_equals_direct_sum(L):
    # Key design 2 of the Caracal notes: the 2L circular convolution truncated to the
    # first L values is the linear causal convolution.
    rng = np.random.default_rng(100 + L)
    v = rng.standard_normal(L)
    g = rng.standard_normal(L)
    r, S = causal_conv_f64(v, g)
    for n in sorted({2 * L, max(1, 2 * L - 1), 1 << (2 * L - 1).bit_length()}):
        c = circular_conv_dft(v, g, n)
        np.testing.assert_allclose(c[:L], r, rtol=0, atol=1e-12 * max(1.0, S.max()))


def test_dft_recipe_matches_numpy_fft():
    rng = np.random.default_rng(3)
    for L, n in ((7, 14), (20, 40), (31, 64)):
        v = rng.standard_normal(L)
        g = rng.standard_normal(L)
        c = circular_conv_dft(v, g, n)
        ref = np.real(np.fft.ifft(np.fft.fft(v, n) * np.fft.fft(g, n)))
        np.testing.assert_allclose(c, ref, rtol=0, atol=1e-11)


@pytest.mark.parametrize("L", [1, 2, 3, 8, 21, 32])
def test_pad_2L_ntt_recipe_equals_exact_sum(L):
    # The exact number-theoretic recipe over Z_p, lifted to the symmetric range, equals
    # the int64 sum bit for bit while |r| <= (p-1)/2.
    rng = np.random.default_rng(200 + L)
    v = rng.integers(-127, 128, size=L)
    g = rng.integers(-127, 128, size=L)
    exact = causal_conv_i64(v, g)
    n = 1 << (2 * L - 1).bit_length() if L > 1 else 2
    c = lift_mod_p(circular_conv_ntt(v, g, n))
    assert np.array_equal(c[:L], exact)
    # negative control: no padding wraps the future around
    if L >= 4:
        n0 = 1 << (L - 1).bit_length()
        if n0 == L:
            w = lift_mod_p(circular_conv_ntt(v, g, L))
            assert not np.array_equal(w[: L - 1], exact[: L - 1])


def test_ntt_recipe_large_values_wrap_mod_p():
    # Beyond |r| <= (p-1)/2 the defined result is the residue: check against Python ints.
    v = np.array([P_NTT - 5, 3, 2**20], dtype=np.int64)
    g = np.array([7, -(2**21), 11], dtype=np.int64)
    ref = [0] * 3
    for t in range(3):
        ref[t] = sum(int(v[j]) * int(g[t - j]) for j in range(t + 1)) % P_NTT
    c = circular_conv_ntt(v, g, 8)
    assert c[:3].tolist() == ref


def test_ntt_constants():
    p = P_NTT
    assert p == 119 * 2**23 + 1
    # p is prime (trial division up to sqrt)
    q = 2
    while q * q <= p:
        assert p % q
        q += 1
    assert (p - 1) == 2**23 * 7 * 17
    # 3 is a primitive root: 3^((p-1)/q) != 1 for each prime q | p-1
    for f in (2, 7, 17):
        assert pow(ROOT_NTT, (p - 1) // f, p) != 1
    for n in (2, 512, 8192, 131072, 2**23):
        w = pow(ROOT_NTT, (p - 1) // n, p)
        assert pow(w, n, p) == 1 and pow(w, n // 2, p) == p - 1
    assert 4 * p < 2**32
    assert (8192 * 998122497) % p == 1


def test_lift():
    p = P_NTT
    r = np.array([0, 1, -1, (p - 1) // 2, -(p - 1) // 2, (p - 1) // 2 + 1, p, 3 * p + 2])
    assert lift_mod_p(r).tolist() == [0, 1, -1, (p - 1) // 2, -(p - 1) // 2, -(p - 1) // 2, 0, 2]


def test_causality_of_oracle():
    rng = np.random.default_rng(11)
    L = 128
    v = rng.standard_normal(L)
    g = rng.standard_normal(L)
    r, _ = causal_conv_f64(v, g)
    for s in (1, 40, 127):
        v2 = v.copy()
        v2[s] += 1.0
        r2, _ = causal_conv_f64(v2, g)
        assert np.array_equal(r2[:s], r[:s])      # bitwise
        assert r2[s] != r[s]                       # g_0 != 0
    vi = rng.integers(-127, 128, size=L)
    gi = rng.integers(-127, 128, size=L)
    gi[0] = 5
    ri = causal_conv_i64(vi, gi)
    vi2 = vi.copy()
    vi2[60] += 3
    ri2 = causal_conv_i64(vi2, gi)
    assert np.array_equal(ri2[:60], ri[:60]) and ri2[60] == ri[60] + 15


def test_sampled_outputs_match_full():
    rng = np.random.default_rng(12)
    v = rng.integers(-50, 50, size=(5, 300)).astype(np.float64)
    g = rng.integers(-50, 50, size=(5, 300)).astype(np.float64)
    r, S = causal_conv_f64(v, g)
    ch = np.array([0, 4, 2, 3, 1, 4])
    t = np.array([0, 299, 150, 1, 77, 0])
    rs, ss = causal_conv_f64_at(v, g, ch, t)
    assert np.array_equal(rs, r[ch, t])       # integer-valued: exact in any order
    assert np.array_equal(ss, S[ch, t])


def test_thread_count_does_not_change_bits():
    rng = np.random.default_rng(13)
    v = rng.standard_normal((13, 257)).astype(np.float32)
    g = rng.standard_normal((13, 257)).astype(np.float32)
    r1, s1 = causal_conv_f64(v, g, nthreads=1)
    r7, s7 = causal_conv_f64(v, g, nthreads=7)
    assert np.array_equal(r1, r7) and np.array_equal(s1, s7)


def test_bf16_decode():
    bits = np.array([0x3F80, 0xC000, 0x3F81, 0x0000, 0x8000, 0x4049], dtype=np.uint16)
    vals = oracle.bf16_bits_to_f64(bits)
    assert vals[0] == 1.0 and vals[1] == -2.0 and vals[2] == 1.0 + 2.0**-7
    assert vals[3] == 0.0 and vals[4] == 0.0 and np.signbit(vals[4])
    assert vals[5] == 3.140625


def test_empty_and_bad_shapes():
    r, S = causal_conv_f64(np.zeros((0, 8)), np.zeros((0, 8)))
    assert r.shape == (0, 8)
    r, S = causal_conv_f64(np.zeros((3, 0)), np.zeros((3, 0)))
    assert r.shape == (3, 0)
    with pytest.raises(ValueError):
        causal_conv_f64(np.zeros((2, 4)), np.zeros((2, 5)))


# ---------------------------------------------------------------- gradients

GOLDEN_BWD = os.path.join(os.path.dirname(__file__), "golden", "hand_cases_bwd.txt")


def _golden_bwd():
    cases = []
    with open(GOLDEN_BWD) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            fields = [x.strip() for x in line.split("|")]
            cases.append((fields[0],) + tuple([int(x) for x in f_.split()] for f_ in fields[1:]))
    assert len(cases) >= 5
    return cases


@pytest.mark.parametrize("case", _golden_bwd(), ids=lambda c: c[0])
def test_golden_bwd(case):
    _, dr, v, g, edv, edg = case
    dv, dg, Sv, Sg = oracle.causal_conv_bwd_f64(np.array(dr, np.float64), np.array(v, np.float64),
                                                np.array(g, np.float64))
    assert dv.tolist() == [float(x) for x in edv]
    assert dg.tolist() == [float(x) for x in edg]
    assert np.all(Sv >= np.abs(dv)) and np.all(Sg >= np.abs(dg))
    idv, idg = oracle.causal_conv_bwd_i64(np.array(dr), np.array(v), np.array(g))
    assert idv.tolist() == edv and idg.tolist() == edg


@pytest.mark.parametrize("L", [1, 2, 3, 17, 64, 200])
def test_bwd_matches_numpy_correlate(L):
    # numpy.correlate(a, b, "full")[L-1+j] = sum_n a[n+j] b[n]: with a = dr, b = g that is dv_j
    rng = np.random.default_rng(500 + L)
    dr, v, g = rng.standard_normal((3, 2, L))
    dv, dg, _, _ = oracle.causal_conv_bwd_f64(dr, v, g)
    for c in range(2):
        np.testing.assert_allclose(dv[c], np.correlate(dr[c], g[c], "full")[L - 1:], rtol=0,
                                   atol=1e-12 * L)
        np.testing.assert_allclose(dg[c], np.correlate(dr[c], v[c], "full")[L - 1:], rtol=0,
                                   atol=1e-12 * L)
    ir, iv, ig = rng.integers(-50, 51, size=(3, 2, L))
    idv, idg = oracle.causal_conv_bwd_i64(ir, iv, ig)
    for c in range(2):
        assert np.array_equal(idv[c], np.correlate(ir[c], ig[c], "full")[L - 1:])
        assert np.array_equal(idg[c], np.correlate(ir[c], iv[c], "full")[L - 1:])


def test_bwd_adjoint_and_reversal_identities_exact():
    # sum_t dr_t r_t = sum_j dv_j v_j = sum_k dg_k g_k (the loss is bilinear), and
    # dv = rev(causal(rev(dr), g)), dg = rev(causal(rev(dr), v)), against the forward oracle
    rng = np.random.default_rng(7)
    for L in (1, 5, 33, 128):
        dr, v, g = rng.integers(-100, 101, size=(3, 3, L))
        r = causal_conv_i64(v, g)
        dv, dg = oracle.causal_conv_bwd_i64(dr, v, g)
        loss = (dr * r).sum(axis=-1)
        assert np.array_equal((dv * v).sum(axis=-1), loss)
        assert np.array_equal((dg * g).sum(axis=-1), loss)
        assert np.array_equal(dv, causal_conv_i64(dr[:, ::-1], g)[:, ::-1])
        assert np.array_equal(dg, causal_conv_i64(dr[:, ::-1], v)[:, ::-1])


def test_bwd_matches_torch_autograd():
    # torch's conv1d (a library convolution) and its autograd, in float64 on the CPU
    import torch
    rng = np.random.default_rng(11)
    nch, L = 3, 40
    dr, v, g = rng.standard_normal((3, nch, L))
    tv = torch.tensor(v, requires_grad=True)
    tg = torch.tensor(g, requires_grad=True)
    # r[c, t] = sum_k g[c, k] v[c, t-k]: cross-correlation of left-padded v with flipped g
    x = torch.nn.functional.pad(tv, (L - 1, 0)).unsqueeze(0)            # (1, nch, 2L-1)
    w = torch.flip(tg, dims=[-1]).unsqueeze(1)                          # (nch, 1, L)
    r = torch.nn.functional.conv1d(x, w, groups=nch)[0]                 # (nch, L)
    (torch.tensor(dr) * r).sum().backward()
    dv, dg, _, _ = oracle.causal_conv_bwd_f64(dr, v, g)
    np.testing.assert_allclose(r.detach().numpy(), causal_conv_f64(v, g)[0], atol=1e-12)
    np.testing.assert_allclose(tv.grad.numpy(), dv, atol=1e-12)
    np.testing.assert_allclose(tg.grad.numpy(), dg, atol=1e-12)


def test_bwd_anticausal_and_scales():
    # dv_j reads dr_t only for t >= j: perturbing dr_s leaves dv_j, dg_j for j > s unchanged
    rng = np.random.default_rng(12)
    L = 50
    dr, v, g = rng.standard_normal((3, L))
    dv, dg, Sv, Sg = oracle.causal_conv_bwd_f64(dr, v, g)
    for s in (0, 17, L - 1):
        d2 = dr.copy()
        d2[s] += 1.0
        dv2, dg2, _, _ = oracle.causal_conv_bwd_f64(d2, v, g)
        assert np.array_equal(dv2[s + 1:], dv[s + 1:]) and np.array_equal(dg2[s + 1:], dg[s + 1:])
        assert dv2[s] != dv[s]
    # the scales are the gradients of the absolute values
    av, ag, _, _ = oracle.causal_conv_bwd_f64(np.abs(dr), np.abs(v), np.abs(g), with_scale=False)
    np.testing.assert_allclose(Sv, av, rtol=1e-14)
    np.testing.assert_allclose(Sg, ag, rtol=1e-14)
    assert np.all(Sv >= np.abs(dv)) and np.all(Sg >= np.abs(dg))
    # threads do not change bits; empty input is fine
    a = oracle.causal_conv_bwd_f64(np.tile(dr, (5, 1)), np.tile(v, (5, 1)), np.tile(g, (5, 1)), nthreads=1)
    b = oracle.causal_conv_bwd_f64(np.tile(dr, (5, 1)), np.tile(v, (5, 1)), np.tile(g, (5, 1)), nthreads=4)
    assert all(np.array_equal(x, y) for x, y in zip(a, b))
    e = oracle.causal_conv_bwd_f64(np.zeros((2, 0)), np.zeros((2, 0)), np.zeros((2, 0)))
    assert e[0].shape == (2, 0)


# ---------------------------------------------------------------- fixed-point exact path

def test_fixed_encode_rounding():
    # nearest, ties to even, on the stored value times 2^f
    x = np.array([0.5, 1.5, 2.5, -0.5, -1.5, 3.25, 0.75, -2.75], dtype=np.float32)
    assert oracle.fixed_encode(x, 0).tolist() == [0, 2, 2, 0, -2, 3, 1, -3]
    assert oracle.fixed_encode(x, 1).tolist() == [1, 3, 5, -1, -3, 6, 2, -6]
    # bf16 bits are decoded exactly: 0x3FC0 = 1.5
    assert oracle.fixed_encode(np.array([0x3FC0], dtype=np.uint16), 3).tolist() == [12]
    with pytest.raises(OverflowError):
        oracle.fixed_encode(np.array([1.0], dtype=np.float32), 62)


def test_int128_sum_against_python_integers():
    rng = np.random.default_rng(41)
    for L in (1, 3, 17):
        v = rng.integers(-2**40, 2**40, size=(2, L), dtype=np.int64)
        g = rng.integers(-2**40, 2**40, size=(2, L), dtype=np.int64)
        r = oracle.causal_conv_i128(v, g)
        for c in range(2):
            for t in range(L):
                assert r[c, t] == sum(int(v[c, j]) * int(g[c, t - j]) for j in range(t + 1))
    small = rng.integers(-1000, 1000, size=(3, 50))
    assert np.array_equal(oracle.causal_conv_i128(small, small[::-1]).astype(np.int64),
                          causal_conv_i64(small, small[::-1]))


def test_rne_to_f32_cases():
    d = oracle.fixed_decode_f32
    # ties to even at the 24-bit boundary, both directions, and negative values
    assert d(np.array([2**24 + 1, 2**24 + 3, -(2**24 + 1)], dtype=object), 0).tolist() == \
        [16777216.0, 16777220.0, -16777216.0]
    # scaling: 3 * 2^-2 exact; 2^25 + 1 at scale 2^-1 rounds to 2^24
    assert d(np.array([3, 2**25 + 1], dtype=object), 2).tolist() == [0.75, 8388608.0]
    # subnormals: smallest, half of it (tie -> 0), three quarters (-> smallest), 1.5x (tie -> 2x)
    sub = np.float32(2.0 ** -149)
    got = d(np.array([1, 3], dtype=object), 149)
    assert oracle._rne_to_f32(1, 149) == float(sub)
    assert oracle._rne_to_f32(1, 150) == 0.0
    assert oracle._rne_to_f32(3, 151) == float(sub)
    assert oracle._rne_to_f32(3, 150) == 2 * float(sub)
    # largest finite float32 and overflow
    fmax = float(np.finfo(np.float32).max)
    assert oracle._rne_to_f32((2**24 - 1) << 104, 0) == fmax
    assert oracle._rne_to_f32(1 << 128, 0) == float("inf")
    assert oracle._rne_to_f32(-(1 << 130), 1) == float("-inf")
    assert got.dtype == np.float32 and got.tolist() == [float(sub), 3 * float(sub)]


def test_rne_to_f32_matches_numpy_single_rounding():
    # for |R| < 2^53 the float64 value R 2^-F is exact, and numpy's float32 cast of it is the
    # one rounding the definition asks for
    rng = np.random.default_rng(42)
    R = [int(x) for x in rng.integers(-2**52, 2**52, size=400)] + [0, 1, -1, 2**52 - 1]
    for F in (0, 7, 30, 60, 130):
        got = oracle.fixed_decode_f32(np.array(R, dtype=object), F)
        want = np.array([np.float32(np.ldexp(float(x), -F)) for x in R], dtype=np.float32)
        assert np.array_equal(got.view(np.uint32), want.view(np.uint32)), F


def test_fixed_path_exact_on_dyadic_inputs():
    # inputs that are exact fixed-point numbers: the encoded sum is the real sum, so the
    # result is that sum rounded once to float32 (the float64 oracle is exact here)
    rng = np.random.default_rng(43)
    fv, fg = 6, 9
    v = (rng.integers(-500, 500, size=(3, 300)) * 2.0 ** -fv).astype(np.float32)
    g = (rng.integers(-500, 500, size=(3, 300)) * 2.0 ** -fg).astype(np.float32)
    r = oracle.causal_conv_fixed_f32(v, g, fv, fg)
    ref, _ = causal_conv_f64(v, g)
    assert np.array_equal(r, ref.astype(np.float32))


def test_fixed_sampled_outputs_match_full():
    # the sampled form against the full 128-bit oracle, with encodings near 2^40 so that the
    # sums pass 2^64 (a sum kept in int64 would wrap) and both tails of each row sampled
    rng = np.random.default_rng(45)
    L, fv, fg = 300, 20, 21
    v = (rng.uniform(-1, 1, size=(4, L)) * 2.0 ** 20).astype(np.float32)
    g = (rng.uniform(-1, 1, size=(4, L)) * 2.0 ** 19).astype(np.float32)
    full = oracle.causal_conv_fixed_f32(v, g, fv, fg)
    R = oracle.causal_conv_i128(oracle.fixed_encode(v, fv), oracle.fixed_encode(g, fg))
    assert max(abs(int(x)) for x in R.ravel()) > 2 ** 64
    ch = np.array([0, 3, 1, 2, 3, 0, 2])
    t = np.array([0, L - 1, 150, 1, 0, L - 1, 299])
    got = oracle.causal_conv_fixed_f32_at(v, g, fv, fg, ch, t)
    assert np.array_equal(got.view(np.uint32), full[ch, t].view(np.uint32))
    with pytest.raises(IndexError):
        oracle.causal_conv_fixed_f32_at(v, g, fv, fg, [4], [0])


def test_fixed_path_error_bound_and_causality():
    rng = np.random.default_rng(44)
    L, fv, fg = 200, 20, 22
    v = rng.standard_normal((2, L)).astype(np.float32)
    g = (1 / (1 + np.exp(-rng.standard_normal((2, L))))).astype(np.float32)
    r = oracle.causal_conv_fixed_f32(v, g, fv, fg)
    ref, _ = causal_conv_f64(v, g)
    # quantization (half a unit of each encoding) plus the final float32 rounding
    cg = np.cumsum(np.abs(g.astype(np.float64)), axis=-1)
    cv = np.cumsum(np.abs(v.astype(np.float64)), axis=-1)
    t = np.arange(1, L + 1)
    bnd = 2.0 ** -(fv + 1) * cg + 2.0 ** -(fg + 1) * cv + t * 2.0 ** -(fv + fg + 2) \
        + 2.0 ** -24 * np.abs(ref)
    assert np.all(np.abs(r - ref) <= bnd)
    for s in (1, 77, L - 1):
        v2 = v.copy()
        v2[:, s] += 0.25
        r2 = oracle.causal_conv_fixed_f32(v2, g, fv, fg)
        assert np.array_equal(r2[:, :s].view(np.uint32), r[:, :s].view(np.uint32))
        assert not np.array_equal(r2[:, s], r[:, s])


def _is_prime(n):
    if n < 2:
        return False
    i = 2
    while i * i <= n:
        if n % i == 0:
            return False
        i += 1
    return True


def test_crt_primes():
    # the three NTT primes the exact real-valued path uses: prime, 2^21 | p - 1, 3 a
    # primitive root, product above 2^88 (the exact range is |R| <= (P - 1) / 2)
    primes = [998244353, 1004535809, 469762049]
    for p in primes:
        assert _is_prime(p)
        assert (p - 1) % (1 << 21) == 0
        m, f = p - 1, 2
        factors = set()
        while f * f <= m:
            while m % f == 0:
                factors.add(f)
                m //= f
            f += 1
        if m > 1:
            factors.add(m)
        assert all(pow(3, (p - 1) // q, p) != 1 for q in factors)
    P = primes[0] * primes[1] * primes[2]
    assert P > 2 ** 88
    # Garner's mixed-radix digits (balanced) reconstruct every R with |R| <= (P-1)/2
    rng = np.random.default_rng(45)
    p0, p1, p2 = primes

    def bal(x, p):
        x %= p
        return x - p if x > (p - 1) // 2 else x

    for R in [0, 1, -1, (P - 1) // 2, -(P - 1) // 2] + [int(x) * 2**60 + int(y) for x, y in
                                                         zip(rng.integers(-2**27, 2**27, 50),
                                                             rng.integers(0, 2**60, 50))]:
        s0, s1, s2 = bal(R, p0), bal(R, p1), bal(R, p2)
        a0 = s0
        a1 = bal((s1 - a0) * pow(p0, -1, p1), p1)
        a2 = bal((s2 - a0 - a1 * p0) * pow(p0 * p1, -1, p2), p2)
        assert a0 + a1 * p0 + a2 * p0 * p1 == R


GOLDEN_FIXED = os.path.join(os.path.dirname(__file__), "golden", "hand_cases_fixed.txt")


def _golden_fixed():
    cases = []
    with open(GOLDEN_FIXED) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            name, fs, v, g, R, r = [x.strip() for x in line.split("|")]
            fv, fg = [int(x) for x in fs.split()]
            cases.append((name, fv, fg, [float(x) for x in v.split()],
                          [float(x) for x in g.split()], [int(x) for x in R.split()],
                          [float(x) for x in r.split()]))
    assert len(cases) >= 3
    return cases


@pytest.mark.parametrize("case", _golden_fixed(), ids=lambda c: c[0])
def test_golden_fixed(case):
    _, fv, fg, v, g, R, r = case
    V = oracle.fixed_encode(np.array(v, np.float32), fv)
    G = oracle.fixed_encode(np.array(g, np.float32), fg)
    assert oracle.causal_conv_i128(V, G).tolist() == R
    assert oracle.causal_conv_fixed_f32(np.array(v, np.float32), np.array(g, np.float32),
                                        fv, fg).tolist() == r


def test_shared_filter_gradients():
    # against torch autograd of a batch of conv1d with one weight per channel (shared by the
    # batch), float64 on the CPU; and the adjoint identity sum dr r = sum dk k exactly on integers
    import torch
    rng = np.random.default_rng(60)
    B, C, L = 3, 2, 30
    dr, v = rng.standard_normal((2, B, C, L))
    k = rng.standard_normal((C, L))
    tv = torch.tensor(v, requires_grad=True)
    tk = torch.tensor(k, requires_grad=True)
    x = torch.nn.functional.pad(tv, (L - 1, 0))                       # (B, C, 2L-1)
    w = torch.flip(tk, dims=[-1]).unsqueeze(1)                        # (C, 1, L)
    r = torch.nn.functional.conv1d(x, w, groups=C)                    # (B, C, L)
    (torch.tensor(dr) * r).sum().backward()
    dv, dk, Sv, Sk = oracle.shared_conv_bwd_f64(dr, v, k)
    np.testing.assert_allclose(tv.grad.numpy(), dv, atol=1e-12)
    np.testing.assert_allclose(tk.grad.numpy(), dk, atol=1e-12)
    assert np.all(Sv >= np.abs(dv)) and np.all(Sk >= np.abs(dk))
    ir = rng.integers(-20, 21, (B, C, L))
    iv = rng.integers(-20, 21, (B, C, L))
    ik = rng.integers(-20, 21, (C, L))
    rr = causal_conv_i64(iv, np.broadcast_to(ik[None], iv.shape))
    _, dki, _, _ = oracle.shared_conv_bwd_f64(ir.astype(float), iv.astype(float), ik.astype(float))
    assert (ir * rr).sum() == int(round((dki * ik).sum()))


# ---------------------------------------------------------------- gate stream

def test_gate_hand_case_zero_padding():
    # s = 0 gives sigma = 1/2 everywhere; W = (1, 2, 3) on taps (t-2, t-1, t).  The padded
    # inputs before t = 0 are zeros of the convolution's input, not sigma(0):
    # g = 1/2 (3, 2+3, 1+2+3, 1+2+3)
    s = np.zeros((1, 1, 4))
    W = np.array([[[1.0, 2.0, 3.0]]])
    g, Sg = oracle.gate_f64(s, W)
    assert np.array_equal(g[0, 0], [1.5, 2.5, 3.0, 3.0])
    assert np.array_equal(Sg, g)


def test_gate_identity_and_shift_taps():
    rng = np.random.default_rng(11)
    B, C, L, cg = 2, 8, 9, 4
    s = rng.standard_normal((B, C, L))
    sig = 1.0 / (1.0 + np.exp(-s))
    for k, shift in ((2, 0), (1, 1), (0, 2)):
        W = np.zeros((C, cg, 3))
        for co in range(C):
            W[co, co % cg, k] = 1.0
        g, _ = oracle.gate_f64(s, W)
        ref = np.zeros_like(sig)
        ref[:, :, shift:] = sig[:, :, :L - shift]
        assert np.array_equal(g, ref), k
    # sigma(x) + sigma(-x) = 1 through the identity tap
    W = np.zeros((C, cg, 3))
    for co in range(C):
        W[co, co % cg, 2] = 1.0
    a, _ = oracle.gate_f64(s, W)
    b, _ = oracle.gate_f64(-s, W)
    np.testing.assert_allclose(a + b, 1.0, rtol=0, atol=1e-15)


def test_gate_against_torch_grouped_conv1d():
    import torch
    rng = np.random.default_rng(12)
    for B, C, L, cg in ((2, 12, 17, 4), (1, 128, 40, 64), (3, 6, 2, 6), (1, 5, 1, 1)):
        s = rng.standard_normal((B, C, L))
        W = rng.standard_normal((C, cg, 3)) / np.sqrt(3.0)
        g, Sg = oracle.gate_f64(s, W)
        x = torch.sigmoid(torch.from_numpy(s))
        x = torch.nn.functional.pad(x, (2, 0))
        ref = torch.nn.functional.conv1d(x, torch.from_numpy(W), groups=C // cg).numpy()
        np.testing.assert_allclose(g, ref, rtol=1e-12, atol=1e-12)
        assert np.all(Sg >= np.abs(g) * (1 - 1e-12))


def test_gate_groups_do_not_mix():
    rng = np.random.default_rng(13)
    B, C, L, cg = 1, 8, 11, 4
    s = rng.standard_normal((B, C, L))
    W = rng.standard_normal((C, cg, 3))
    g, _ = oracle.gate_f64(s, W)
    s2 = s.copy()
    s2[:, cg:] += 1.0                       # the second group's inputs
    g2, _ = oracle.gate_f64(s2, W)
    assert np.array_equal(g[:, :cg], g2[:, :cg])
    assert not np.array_equal(g[:, cg:], g2[:, cg:])
    # bf16 storage is decoded exactly: the same values as float64 inputs
    from workloads import f32_to_bf16_bits
    sb = f32_to_bf16_bits(s.astype(np.float32))
    gb, _ = oracle.gate_f64(sb, W)
    gd, _ = oracle.gate_f64(oracle.as_f64(sb), W)
    assert np.array_equal(gb, gd)
