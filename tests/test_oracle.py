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
