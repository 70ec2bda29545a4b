"""Seeded synthetic inputs for the causal long convolution.

This module is shared by the oracle side (tests, cpu baseline) and the GPU side (tests,
smoke check, bench) and therefore holds none of the convolution's arithmetic: it only
draws random numbers, shapes them like the pages' models and rounds them to the stored
dtype.  Every array is generated in float64 from ``numpy.random.default_rng`` seeded with
``SeedSequence([config_id, stream_id])`` (stream 0 = v, 1 = gate pre-activation,
2 = gate conv weights, 3 = extra draws such as perturbation positions, 4 = the upstream
gradient dr of the backward pass, 5 = a filter shared by the batch), then rounded once to
the stored dtype.

Workload shapes (the model shapes follow "Caracal: Causal Architecture via Spectral
Mixing": the multi-head Fourier module mixes C = n_head * head_dim channels per batch
element, with a data-dependent gate stream produced by a grouped Conv1d over sigma(.) of a
projection; main and ablation tables give the model sizes and the 4096 context):

=====  ==========  ====  =====  ======  ====================================================
 id     B           C     L      store   g
=====  ==========  ====  =====  ======  ====================================================
 1     1           64    256    fp32    sigmoid(N(0,1))
 2     8           768   1024   fp32    grouped causal conv k=3 (12 groups of 64),
                                        W ~ N(0, variance 1/3), of sigmoid(N(0,1))
 3     8           1024  4096   bf16    as 2 with 16 groups
 4     1           1536  65536  fp32    sigmoid(N(0,1)) * exp(-t / 16384)
 5     4           768   4096   int32   uniform integers in [-127, 127] (v likewise)
 6     8           1024  4096   fp32    the draws of 3 (same seeds) stored as fp32
 7     1           1536  65536  int32   uniform integers in [-127, 127] (v likewise): the
                                        long-context shape of 4 for the exact kind
=====  ==========  ====  =====  ======  ====================================================

For 1-4, v ~ N(0,1).  The datasets the pages evaluate on are not used; these synthetic
tensors stand in for the activations of those models.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np


@dataclass(frozen=True)
class Workload:
    cid: int
    name: str
    B: int
    C: int
    L: int
    storage: str      # "f32" | "bf16" | "i32"
    gate: str         # "sigmoid" | "conv" | "decay" | "int"
    groups: int = 0   # for gate == "conv"

    @property
    def channels(self) -> int:
        return self.B * self.C

    @property
    def outputs(self) -> int:
        return self.B * self.C * self.L


WORKLOADS = {
    1: Workload(1, "tiny-f32-B1-C64-L256", 1, 64, 256, "f32", "sigmoid"),
    2: Workload(2, "small-mhf-f32-B8-C768-L1024", 8, 768, 1024, "f32", "conv", 12),
    3: Workload(3, "medium-mhf-bf16-B8-C1024-L4096", 8, 1024, 4096, "bf16", "conv", 16),
    4: Workload(4, "long-fourstep-f32-B1-C1536-L65536", 1, 1536, 65536, "f32", "decay"),
    5: Workload(5, "ntt-i32-B4-C768-L4096", 4, 768, 4096, "i32", "int"),
    # the Medium shape with fp32 storage: same seeds (cid 3) as workload 3
    6: Workload(3, "medium-mhf-f32-B8-C1024-L4096", 8, 1024, 4096, "f32", "conv", 16),
    # the long-context shape with the exact workload's integers (four-step NTT)
    7: Workload(7, "long-exact-i32-B1-C1536-L65536", 1, 1536, 65536, "i32", "int"),
}


def rng(cid: int, stream: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([int(cid), int(stream)]))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest, ties to even); return the bits
    as uint16.  Inputs must be finite."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (b >> np.uint32(16)) & np.uint32(1)
    return ((b + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact decode of bfloat16 bits to float32."""
    return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32)
            << np.uint32(16)).view(np.float32)


def _sigmoid(x: np.ndarray) -> np.ndarray:
    return 1.0 / (1.0 + np.exp(-x))


def _grouped_causal_conv3(s: np.ndarray, w: np.ndarray, groups: int) -> np.ndarray:
    """Gate synthesis (input recipe only, not the convolution under test):
    out[b, co, t] = sum_{ci in group(co)} sum_{k=0..2} w[co, ci - c0, k] * s[b, ci, t + k - 2]
    with s[..., tau < 0] = 0 (causal left padding of 2, PyTorch tap order)."""
    B, C, L = s.shape
    cg = C // groups
    wg = w.reshape(groups, cg, cg, 3)
    taps = [np.ascontiguousarray(wg[:, :, :, k]) for k in range(3)]
    out = np.empty((B, C, L), dtype=np.float64)
    for b in range(B):
        for gi in range(groups):
            blk = s[b, gi * cg:(gi + 1) * cg]          # (cg, L) inputs of this group
            acc = taps[2][gi] @ blk                     # tap k=2 reads s[t]
            if L > 1:
                acc[:, 1:] += taps[1][gi] @ blk[:, :-1]  # tap k=1 reads s[t-1]
            if L > 2:
                acc[:, 2:] += taps[0][gi] @ blk[:, :-2]  # tap k=0 reads s[t-2]
            out[b, gi * cg:(gi + 1) * cg] = acc
    return out


def make_inputs(w: Workload, B: int | None = None, C: int | None = None,
                L: int | None = None, seed_offset: int = 0):
    """Inputs ``(v, g)`` of shape (B, C, L) in the workload's stored dtype:
    float32, uint16 bf16 bits, or int32.  ``B``, ``C``, ``L`` override the shape while
    keeping the workload's distributions (used for small parity cases); ``seed_offset``
    selects a different seed family."""
    B = w.B if B is None else B
    C = w.C if C is None else C
    L = w.L if L is None else L
    cid = w.cid + 1000 * seed_offset
    shape = (B, C, L)
    if w.gate == "int":
        v = rng(cid, 0).integers(-127, 128, size=shape, dtype=np.int32)
        g = rng(cid, 1).integers(-127, 128, size=shape, dtype=np.int32)
        return v, g
    v64 = rng(cid, 0).standard_normal(shape)
    pre = rng(cid, 1).standard_normal(shape)
    if w.gate == "sigmoid":
        g64 = _sigmoid(pre)
    elif w.gate == "decay":
        g64 = _sigmoid(pre) * np.exp(-np.arange(L, dtype=np.float64) / 16384.0)
    elif w.gate == "conv":
        groups = w.groups
        if C % groups:
            groups = 1
        cg = C // groups
        wts = rng(cid, 2).standard_normal((C, cg, 3)) * np.sqrt(1.0 / 3.0)
        g64 = _grouped_causal_conv3(_sigmoid(pre), wts, groups)
    else:
        raise ValueError(w.gate)
    v32 = v64.astype(np.float32)
    g32 = g64.astype(np.float32)
    if w.storage == "bf16":
        return f32_to_bf16_bits(v32), f32_to_bf16_bits(g32)
    return v32, g32


def make_gate_inputs(w: Workload, B: int | None = None, C: int | None = None,
                     L: int | None = None, seed_offset: int = 0, cg: int = 64):
    """Inputs ``(v, s, W)`` of the gate-stream calls, in the workload's float storage: v
    (B, C, L) as :func:`make_inputs`, the gate pre-activation s (B, C, L) ~ N(0, 1) and the
    grouped kernel-3 weights W (C, cg, 3) ~ N(0, variance 1/3) (the same streams 0, 1, 2)."""
    if w.storage not in ("f32", "bf16"):
        raise ValueError("the gate calls take float storage")
    B = w.B if B is None else B
    C = w.C if C is None else C
    L = w.L if L is None else L
    cid = w.cid + 1000 * seed_offset
    shape = (B, C, L)
    v32 = rng(cid, 0).standard_normal(shape).astype(np.float32)
    s32 = rng(cid, 1).standard_normal(shape).astype(np.float32)
    w32 = (rng(cid, 2).standard_normal((C, cg, 3)) * np.sqrt(1.0 / 3.0)).astype(np.float32)
    if w.storage == "bf16":
        return f32_to_bf16_bits(v32), f32_to_bf16_bits(s32), f32_to_bf16_bits(w32)
    return v32, s32, w32


def make_grad(w: Workload, B: int | None = None, C: int | None = None, L: int | None = None,
              seed_offset: int = 0) -> np.ndarray:
    """Upstream gradient ``dr`` = dLoss/dr for the backward pass, shape (B, C, L) in the
    workload's stored dtype: N(0,1) for the float workloads (the gradient of a next-token
    loss reaching the mixer has no structure to imitate here), uniform integers in
    [-127, 127] for the exact workload."""
    B = w.B if B is None else B
    C = w.C if C is None else C
    L = w.L if L is None else L
    cid = w.cid + 1000 * seed_offset
    shape = (B, C, L)
    if w.gate == "int":
        return rng(cid, 4).integers(-127, 128, size=shape, dtype=np.int32)
    d32 = rng(cid, 4).standard_normal(shape).astype(np.float32)
    return f32_to_bf16_bits(d32) if w.storage == "bf16" else d32


def make_shared_filter(w: Workload, C: int | None = None, L: int | None = None,
                       seed_offset: int = 0) -> np.ndarray:
    """A filter per channel, shared by every batch row, shape (C, L), in the workload's
    stored dtype: k[c][t] = N(0,1) * exp(-t / tau_c) with tau_c log-spaced over [16, L]
    (a decaying long filter like the position-based filters the Caracal notes contrast with
    their data-dependent gate).  Drawn from stream 5."""
    C = w.C if C is None else C
    L = w.L if L is None else L
    cid = w.cid + 1000 * seed_offset
    tau = np.exp(np.linspace(np.log(16.0), np.log(max(L, 17)), C))[:, None]
    k64 = rng(cid, 5).standard_normal((C, L)) * np.exp(-np.arange(L)[None, :] / tau)
    k32 = k64.astype(np.float32)
    return f32_to_bf16_bits(k32) if w.storage == "bf16" else k32


def perturbation_positions(cid: int, L: int, count: int = 8) -> np.ndarray:
    """Seeded positions s for the future-token leakage probe; always includes 1 and
    L-1 (when L > 1)."""
    r = rng(cid, 3)
    pos = {1, L - 1} if L > 1 else {0}
    extra = r.integers(1, max(L, 2), size=4 * count)
    for p in extra:
        if len(pos) >= count:
            break
        pos.add(int(p) % L)
    return np.array(sorted(pos), dtype=np.int64)
