"""Helpers shared by the GPU tests: device transfer and the parity bounds.

Bounds (float kinds), per output t of every channel:
    fp32:  |r - r_ref| <= 1e-4 * S_t,              S_t = sum_{j<=t} |v_j| |g_{t-j}|
    bf16:  |r - r_ref| <= 1e-4 * S_t + 2^-8 * (|r_ref| + 1e-4 * S_t)
The second term of the bf16 bound is the one final rounding to bfloat16 (unit round-off
2^-8) of a value that is itself within the fp32 bound.  r_ref and S come from the float64
oracle on the stored (already rounded) inputs.
"""
from __future__ import annotations

import numpy as np
import torch

TOL = 1e-4


def to_device(x: np.ndarray, dev="cuda:0") -> torch.Tensor:
    if x.dtype == np.uint16:          # bfloat16 bit patterns
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).to(dev).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(x)).to(dev)


def to_host(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def decode(x: np.ndarray) -> np.ndarray:
    """Stored values -> float64 (bf16 bits decoded exactly)."""
    if x.dtype == np.uint16:
        return (x.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    return x.astype(np.float64)


def bound(r_ref: np.ndarray, S: np.ndarray, bf16: bool) -> np.ndarray:
    b = TOL * S
    if bf16:
        b = b + 2.0 ** -8 * (np.abs(r_ref) + b)
    return b


def assert_within_bound(r_gpu: np.ndarray, r_ref: np.ndarray, S: np.ndarray, bf16: bool,
                        what: str = "") -> float:
    """Assert the per-output bound; return the worst err/bound ratio."""
    r = decode(r_gpu)
    err = np.abs(r - r_ref)
    b = bound(r_ref, S, bf16)
    bad = err > b
    with np.errstate(divide="ignore", invalid="ignore"):
        ratio = np.where(b > 0, err / b, np.where(err > 0, np.inf, 0.0))
    worst = float(ratio.max()) if ratio.size else 0.0
    if bad.any():
        idx = np.unravel_index(int(np.argmax(ratio)), ratio.shape)
        raise AssertionError(
            "%s: %d of %d outputs outside the bound; worst ratio %.3g at %s "
            "(gpu %r, ref %r, S %r)" % (what, int(bad.sum()), bad.size, worst, idx,
                                        float(r[idx]), float(r_ref[idx]), float(S[idx])))
    return worst
