"""CPU oracle for the batched causal long convolution -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py``
may import this package.  The product path (``fft_causal_long_amd`` / libspecconv) never
imports, links or calls it, and the two share no code: this package does its own
storage decoding (bf16 bits -> float), its own modular lift and its own builds.

Every function is a plain definition or the pages' recipe written out without any
blocking or fusion (see ``oracle.c`` for the C side):

* :func:`causal_conv_f64` -- r[t] = sum_{j<=t} v[j] g[t-j] and the error scale
  S[t] = sum_{j<=t} |v[j]| |g[t-j]|, float64.  This is the causal convolution that
  "Caracal: Causal Architecture via Spectral Mixing" (key design 1, the multi-head
  Fourier module) equates with the frequency-domain product, and that key design 2
  (the frequency-domain causal mask) says pad-to-2L / truncate-to-L reduces to.
* :func:`causal_conv_i64` -- the same sum in exact int64.
* :func:`lift_mod_p` -- residue of an exact integer, mapped to the symmetric range
  [-(p-1)/2, (p-1)/2]: what an exact number-theoretic transform returns ("Catastrophic
  Token Leakage in Convolutional Sequence Modeling and How to Mitigate It", abstract:
  FFTs done on integers only).
* :func:`causal_conv_f64_at` -- the float64 sum for sampled (channel, t) outputs.
* :func:`shared_conv_bwd_f64` -- the same gradients for a filter shared by the batch: dv
  per row, dk summed over the batch rows (the filter is one parameter for all of them).
* :func:`causal_conv_bwd_f64` / :func:`causal_conv_bwd_i64` -- the gradients of
  sum_t dr[t] r[t]: dv[j] = sum_{t>=j} dr[t] g[t-j], dg[k] = sum_{t>=k} dr[t] v[t-k], with
  their error scales (the pages' models are trained end to end with a next-token loss,
  "Caracal", loss function / training strategy).
* :func:`fixed_encode`, :func:`causal_conv_i128`, :func:`fixed_decode_f32`,
  :func:`causal_conv_fixed_f32` -- the exactly causal real-valued convolution: inputs
  encoded as integers V = round(v 2^fv), G = round(g 2^fg) (nearest, ties to even), the
  exact integer causal sum R (signed 128-bit), and r = R 2^-(fv+fg) rounded once to
  float32 (nearest, ties to even, subnormals included).  The leakage page proposes
  transforms executed on integers only ("Catastrophic Token Leakage ...", abstract); a
  fixed-point encoding with caller-chosen scales carries real activations onto integers
  without letting any output depend on a later input.  :func:`causal_conv_fixed_f32_at`
  gives the same result at sampled outputs, each sum formed in Python integers.
* :func:`gate_f64` -- the gate stream of the multi-head Fourier module ("Caracal", key
  design 1): a causal convolution with kernel 3 over sigma(s), grouped by head (the
  channels of one group mix with each other only), g[co, t] = sum_{i, k} W[co, i, k]
  sigma(s[c0 + i, t + k - 2]) with the convolution's input zero before t = 0, and its error
  scale sum |W| sigma(s).
* :func:`circular_conv_dft` / :func:`circular_conv_ntt` -- the pages' recipe (zero-pad on
  the right to n, transform, multiply, inverse, keep all n values) with O(n^2) DFT / NTT,
  used only to pin key design 2 against the direct sum.

NTT modulus: p = 998244353 = 119 * 2^23 + 1 with primitive root 3.  The pages fix only
"32-bit integers"; this prime is the reading used on both sides of the parity tests.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

P_NTT = 998244353
ROOT_NTT = 3

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lock = threading.Lock()
_lib = None


def build(force: bool = False) -> str:
    """Compile oracle.c with gcc into oracle/liboracle.so (host code only)."""
    if force or not os.path.exists(_LIB_PATH) or (
        os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC)
    ):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        cmd = [
            "gcc", "-O2", "-ffp-contract=off", "-fPIC", "-shared", "-std=c99",
            "-Wall", "-o", tmp, _SRC, "-lm", "-lpthread",
        ]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(_LIB_PATH) or (
            os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC)
        ):
            build()
        lib = ctypes.CDLL(_LIB_PATH)
        i64, dp, lp = ctypes.c_int64, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int64)
        lib.oracle_conv_f64.argtypes = [dp, dp, dp, dp, i64, i64, ctypes.c_int]
        lib.oracle_conv_f64.restype = ctypes.c_int
        lib.oracle_conv_i64.argtypes = [lp, lp, lp, i64, i64, ctypes.c_int]
        lib.oracle_conv_i64.restype = ctypes.c_int
        lib.oracle_conv_f64_at.argtypes = [dp, dp, i64, lp, lp, i64, dp, dp]
        lib.oracle_conv_f64_at.restype = ctypes.c_int
        lib.oracle_circular_dft_f64.argtypes = [dp, dp, i64, i64, dp]
        lib.oracle_circular_dft_f64.restype = ctypes.c_int
        lib.oracle_circular_ntt.argtypes = [lp, lp, i64, i64, ctypes.c_uint32, ctypes.c_uint32, lp]
        lib.oracle_circular_ntt.restype = ctypes.c_int
        lib.oracle_conv_bwd_f64.argtypes = [dp] * 7 + [i64, i64, ctypes.c_int]
        lib.oracle_conv_bwd_f64.restype = ctypes.c_int
        lib.oracle_conv_bwd_i64.argtypes = [lp] * 5 + [i64, i64, ctypes.c_int]
        lib.oracle_conv_i128.argtypes = [lp, lp, lp, ctypes.POINTER(ctypes.c_uint64), i64, i64,
                                         ctypes.c_int]
        lib.oracle_conv_i128.restype = ctypes.c_int
        lib.oracle_conv_bwd_i64.restype = ctypes.c_int
        _lib = lib
        return lib


def _dptr(a):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def _lptr(a):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_int64))


def default_threads() -> int:
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return max(1, os.cpu_count() or 1)


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Decode stored bfloat16 bit patterns (uint16) exactly: bf16 is the top half of an
    IEEE binary32, so shifting the bits up gives the float32 with the same value."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def as_f64(x: np.ndarray) -> np.ndarray:
    """Widen stored values exactly to float64 (uint16 arrays are read as bf16 bits)."""
    x = np.asarray(x)
    if x.dtype == np.uint16:
        return bf16_bits_to_f64(x)
    if x.dtype not in (np.float16, np.float32, np.float64):
        raise TypeError("oracle: unsupported float storage dtype %s" % x.dtype)
    return np.ascontiguousarray(x, dtype=np.float64)


def causal_conv_f64(v, g, nthreads: int | None = None, with_scale: bool = True):
    """Direct float64 causal convolution along the last axis.

    Returns ``(r, S)`` (``S`` is None when ``with_scale`` is False); both have the
    shape of ``v``.  Inputs are widened exactly from their stored dtype."""
    v64, g64 = as_f64(v), as_f64(g)
    if v64.shape != g64.shape:
        raise ValueError("v and g must have the same shape")
    shape = v64.shape
    L = shape[-1] if len(shape) else 0
    nch = int(np.prod(shape[:-1])) if len(shape) > 1 else 1
    r = np.zeros(shape, dtype=np.float64)
    S = np.zeros(shape, dtype=np.float64) if with_scale else None
    if v64.size == 0:
        return r, S
    rc = _load().oracle_conv_f64(
        _dptr(v64), _dptr(g64), _dptr(r), _dptr(S) if S is not None else None,
        nch, L, nthreads or default_threads(),
    )
    if rc != 0:
        raise RuntimeError("oracle_conv_f64 failed")
    return r, S


def causal_conv_i64(v, g, nthreads: int | None = None) -> np.ndarray:
    """Exact int64 causal convolution along the last axis."""
    v64 = np.ascontiguousarray(v, dtype=np.int64)
    g64 = np.ascontiguousarray(g, dtype=np.int64)
    if v64.shape != g64.shape:
        raise ValueError("v and g must have the same shape")
    shape = v64.shape
    L = shape[-1] if len(shape) else 0
    nch = int(np.prod(shape[:-1])) if len(shape) > 1 else 1
    r = np.zeros(shape, dtype=np.int64)
    if v64.size == 0:
        return r
    rc = _load().oracle_conv_i64(_lptr(v64), _lptr(g64), _lptr(r), nch, L,
                                 nthreads or default_threads())
    if rc != 0:
        raise RuntimeError("oracle_conv_i64 failed")
    return r


def causal_conv_bwd_f64(dr, v, g, nthreads: int | None = None, with_scale: bool = True):
    """Gradients of sum_t dr[t] r[t] for the causal convolution r of v and g (last axis),
    float64: returns ``(dv, dg, Sv, Sg)`` with Sv[j] = sum_{t>=j} |dr[t]| |g[t-j]| and Sg
    likewise (both None when ``with_scale`` is False)."""
    d64, v64, g64 = as_f64(dr), as_f64(v), as_f64(g)
    if not (d64.shape == v64.shape == g64.shape):
        raise ValueError("dr, v and g must have the same shape")
    shape = v64.shape
    L = shape[-1] if len(shape) else 0
    nch = int(np.prod(shape[:-1])) if len(shape) > 1 else 1
    dv, dg = np.zeros(shape), np.zeros(shape)
    Sv = np.zeros(shape) if with_scale else None
    Sg = np.zeros(shape) if with_scale else None
    if v64.size == 0:
        return dv, dg, Sv, Sg
    rc = _load().oracle_conv_bwd_f64(
        _dptr(d64), _dptr(v64), _dptr(g64), _dptr(dv), _dptr(dg),
        _dptr(Sv) if with_scale else None, _dptr(Sg) if with_scale else None,
        nch, L, nthreads or default_threads(),
    )
    if rc != 0:
        raise RuntimeError("oracle_conv_bwd_f64 failed")
    return dv, dg, Sv, Sg


def causal_conv_bwd_i64(dr, v, g, nthreads: int | None = None):
    """Exact int64 gradients ``(dv, dg)`` of sum_t dr[t] r[t] (last axis)."""
    d64 = np.ascontiguousarray(dr, dtype=np.int64)
    v64 = np.ascontiguousarray(v, dtype=np.int64)
    g64 = np.ascontiguousarray(g, dtype=np.int64)
    if not (d64.shape == v64.shape == g64.shape):
        raise ValueError("dr, v and g must have the same shape")
    shape = v64.shape
    L = shape[-1] if len(shape) else 0
    nch = int(np.prod(shape[:-1])) if len(shape) > 1 else 1
    dv, dg = np.zeros(shape, dtype=np.int64), np.zeros(shape, dtype=np.int64)
    if v64.size == 0:
        return dv, dg
    rc = _load().oracle_conv_bwd_i64(_lptr(d64), _lptr(v64), _lptr(g64), _lptr(dv), _lptr(dg),
                                     nch, L, nthreads or default_threads())
    if rc != 0:
        raise RuntimeError("oracle_conv_bwd_i64 failed")
    return dv, dg


def fixed_encode(x, f: int) -> np.ndarray:
    """V = round(x * 2^f) (nearest, ties to even) as int64, exact: x is widened exactly from
    its stored dtype, the power-of-two scaling is exact in float64, and numpy.rint rounds
    half to even.  Raises OverflowError when some |x 2^f| reaches 2^62."""
    y = np.ldexp(as_f64(x), int(f))
    if y.size and not np.all(np.abs(y) < 2.0 ** 62):
        raise OverflowError("fixed_encode: |x * 2^f| >= 2^62")
    return np.rint(y).astype(np.int64)


def causal_conv_i128(V, G, nthreads: int | None = None) -> np.ndarray:
    """Exact causal sum of int64 sequences in 128-bit arithmetic; returns Python integers
    (numpy object array of the input shape)."""
    v64 = np.ascontiguousarray(V, dtype=np.int64)
    g64 = np.ascontiguousarray(G, dtype=np.int64)
    if v64.shape != g64.shape:
        raise ValueError("V and G must have the same shape")
    shape = v64.shape
    L = shape[-1] if len(shape) else 0
    nch = int(np.prod(shape[:-1])) if len(shape) > 1 else 1
    hi = np.zeros(shape, dtype=np.int64)
    lo = np.zeros(shape, dtype=np.uint64)
    if v64.size:
        rc = _load().oracle_conv_i128(_lptr(v64), _lptr(g64), _lptr(hi),
                                      lo.ctypes.data_as(ctypes.POINTER(ctypes.c_uint64)),
                                      nch, L, nthreads or default_threads())
        if rc != 0:
            raise RuntimeError("oracle_conv_i128 failed")
    out = np.empty(shape, dtype=object)
    flat_hi, flat_lo, flat = hi.ravel(), lo.ravel(), out.reshape(-1)
    for i in range(flat.size):
        flat[i] = (int(flat_hi[i]) << 64) + int(flat_lo[i])
    return out


def _rne_to_f32(R: int, F: int) -> float:
    """The float32 nearest to R * 2^-F (ties to even; subnormals; overflow to inf)."""
    if R == 0:
        return 0.0
    m = -R if R < 0 else R
    e = m.bit_length() - 1 - F                  # R 2^-F lies in [2^e, 2^(e+1))
    qexp = max(e - 23, -149)                    # spacing of float32 numbers there
    sh = F + qexp                               # keep m / 2^sh, rounded to an integer
    if sh <= 0:
        mant = m << (-sh)
    else:
        mant = m >> sh
        rem = m - (mant << sh)
        half = 1 << (sh - 1)
        if rem > half or (rem == half and (mant & 1)):
            mant += 1
    if mant >= (1 << 24) and qexp + 24 > 128:   # rounds past the largest finite float32
        val = float("inf")
    else:
        val = float(mant) * 2.0 ** qexp          # exact in float64
        if val >= 2.0 ** 128:
            val = float("inf")
    return -val if R < 0 else val


def fixed_decode_f32(R, F: int) -> np.ndarray:
    """Round each exact integer R (object array) times 2^-F once to float32."""
    R = np.asarray(R, dtype=object)
    out = np.empty(R.shape, dtype=np.float32)
    flat, o = R.reshape(-1), out.reshape(-1)
    for i in range(flat.size):
        o[i] = np.float32(_rne_to_f32(int(flat[i]), int(F)))
    return out


def causal_conv_fixed_f32(v, g, fv: int, fg: int, nthreads: int | None = None) -> np.ndarray:
    """The exactly causal real-valued convolution: float32 result of
    round_f32(sum_{j<=t} round(v_j 2^fv) round(g_{t-j} 2^fg) * 2^-(fv+fg))."""
    return fixed_decode_f32(causal_conv_i128(fixed_encode(v, fv), fixed_encode(g, fg),
                                             nthreads), fv + fg)


def causal_conv_fixed_f32_at(v, g, fv: int, fg: int, ch, t) -> np.ndarray:
    """causal_conv_fixed_f32 at sampled outputs r[ch[i], t[i]] of (nch, L) inputs: the same
    definition, each exact sum R_t = sum_{j<=t} V_j G_{t-j} formed in Python integers one
    output at a time (for lengths where the full 128-bit convolution is too slow)."""
    V, G = fixed_encode(v, fv), fixed_encode(g, fg)
    if V.shape != G.shape:
        raise ValueError("v and g must have the same shape")
    L = V.shape[-1]
    V, G = V.reshape(-1, L), G.reshape(-1, L)
    ch = np.asarray(ch, dtype=np.int64).ravel()
    t = np.asarray(t, dtype=np.int64).ravel()
    if ch.shape != t.shape:
        raise ValueError("ch and t must have the same shape")
    out = np.empty(ch.shape, dtype=np.float32)
    for i in range(ch.size):
        c, tt = int(ch[i]), int(t[i])
        if not (0 <= c < V.shape[0] and 0 <= tt < L):
            raise IndexError("sample out of range")
        R = int(np.dot(V[c, :tt + 1].astype(object), G[c, tt::-1].astype(object)))
        out[i] = np.float32(_rne_to_f32(R, int(fv) + int(fg)))
    return out


def shared_conv_bwd_f64(dr, v, k, nthreads: int | None = None):
    """Gradients for a filter shared by the batch, r[b, c] = causal(v[b, c], k[c]):
    dv[b, c, j] = sum_{t>=j} dr[b, c, t] k[c, t-j] and dk[c, j] = sum_b sum_{t>=j}
    dr[b, c, t] v[b, c, t-j] (the batch sum of the per-row gradient), float64, with their
    error scales.  dr, v: (B, C, L); k: (C, L).  Returns (dv, dk, Sv, Sk)."""
    d64, v64, k64 = as_f64(dr), as_f64(v), as_f64(k)
    if d64.shape != v64.shape or v64.ndim != 3 or k64.shape != v64.shape[1:]:
        raise ValueError("dr, v must be (B, C, L) and k (C, L)")
    kb = np.ascontiguousarray(np.broadcast_to(k64[None], v64.shape))
    dv, dkb, Sv, Skb = causal_conv_bwd_f64(d64, v64, kb, nthreads)
    return dv, dkb.sum(axis=0), Sv, Skb.sum(axis=0)


def gate_f64(s, W):
    """Gate stream g = Conv1d_G2(sigma(s)), float64, with its error scale.

    s: (B, C, L) pre-activation (stored values, decoded exactly); W: (C, cg, 3) weights of a
    convolution grouped into C / cg groups of cg channels, PyTorch's tap order (tap k
    multiplies the input at t + k - 2, i.e. causal left padding by 2 of sigma(s), the padded
    entries being 0).  Returns (g, Sg) with Sg[b, co, t] = sum_{i, k} |W[co, i, k]|
    sigma(s[b, c0 + i, t + k - 2]), where c0 is the first channel of co's group."""
    s64, w64 = as_f64(s), as_f64(W)
    if s64.ndim != 3 or w64.ndim != 3 or w64.shape[2] != 3 or w64.shape[0] != s64.shape[1]:
        raise ValueError("s must be (B, C, L) and W (C, cg, 3)")
    B, C, L = s64.shape
    cg = w64.shape[1]
    if cg < 1 or C % cg:
        raise ValueError("the group size must divide C")
    sig = 1.0 / (1.0 + np.exp(-s64))
    # the convolution's input, zero at t = -2, -1
    padded = np.concatenate([np.zeros((B, C, 2)), sig], axis=2)
    g = np.zeros((B, C, L))
    Sg = np.zeros((B, C, L))
    for c0 in range(0, C, cg):
        wg = w64[c0:c0 + cg]                                  # (cg out, cg in, 3)
        for k in range(3):
            x = padded[:, c0:c0 + cg, k:k + L]                 # input at t + k - 2
            g[:, c0:c0 + cg] += np.matmul(wg[:, :, k], x)
            Sg[:, c0:c0 + cg] += np.matmul(np.abs(wg[:, :, k]), x)
    return g, Sg


def lift_mod_p(r, p: int = P_NTT) -> np.ndarray:
    """(r mod p) mapped into [-(p-1)/2, (p-1)/2] (p odd, so there is no tie)."""
    r = np.asarray(r, dtype=np.int64)
    m = np.mod(r, p)
    return np.where(m > (p - 1) // 2, m - p, m).astype(np.int64)


def causal_conv_f64_at(v, g, ch, t):
    """float64 r and S at sampled outputs: v, g of shape (nch, L); ch, t index arrays."""
    v64, g64 = as_f64(v), as_f64(g)
    L = v64.shape[-1]
    v64 = v64.reshape(-1, L)
    g64 = g64.reshape(-1, L)
    ch = np.ascontiguousarray(ch, dtype=np.int64)
    t = np.ascontiguousarray(t, dtype=np.int64)
    if ch.shape != t.shape:
        raise ValueError("ch and t must have the same shape")
    if ch.size and (ch.min() < 0 or ch.max() >= v64.shape[0]):
        raise IndexError("channel index out of range")
    r = np.zeros(ch.shape, dtype=np.float64)
    S = np.zeros(ch.shape, dtype=np.float64)
    rc = _load().oracle_conv_f64_at(_dptr(v64), _dptr(g64), L, _lptr(ch), _lptr(t), ch.size,
                                    _dptr(r), _dptr(S))
    if rc != 0:
        raise RuntimeError("oracle_conv_f64_at failed")
    return r, S


def circular_conv_dft(v, g, n: int) -> np.ndarray:
    """Naive O(n^2) float64 DFT circular convolution of v, g zero-padded to n (1-D)."""
    v64 = np.ascontiguousarray(v, dtype=np.float64).ravel()
    g64 = np.ascontiguousarray(g, dtype=np.float64).ravel()
    if v64.size != g64.size:
        raise ValueError("v and g must have the same length")
    out = np.zeros(n, dtype=np.float64)
    rc = _load().oracle_circular_dft_f64(_dptr(v64), _dptr(g64), v64.size, n, _dptr(out))
    if rc != 0:
        raise RuntimeError("oracle_circular_dft_f64 failed")
    return out


def circular_conv_ntt(v, g, n: int, p: int = P_NTT, root: int = ROOT_NTT) -> np.ndarray:
    """Naive O(n^2) NTT circular convolution mod p of v, g zero-padded to n (1-D).
    Returns residues in [0, p)."""
    v64 = np.ascontiguousarray(v, dtype=np.int64).ravel()
    g64 = np.ascontiguousarray(g, dtype=np.int64).ravel()
    if v64.size != g64.size:
        raise ValueError("v and g must have the same length")
    out = np.zeros(n, dtype=np.int64)
    rc = _load().oracle_circular_ntt(_lptr(v64), _lptr(g64), v64.size, n, p, root, _lptr(out))
    if rc != 0:
        raise RuntimeError("oracle_circular_ntt failed")
    return out
