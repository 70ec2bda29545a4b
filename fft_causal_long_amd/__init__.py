"""fft_causal_long_amd -- Python binding of libspecconv (argument marshalling only).

The batched per-channel causal long convolution

    r[b, c, t] = sum_{j <= t} v[b, c, j] * g[b, c, t - j]

runs entirely in the HIP kernels of ``libspecconv.so`` (built in-tree from ``csrc/`` by
``python -m fft_causal_long_amd.build``).  PyTorch only provides device memory and the
stream: tensors are passed by ``data_ptr()`` together with the current HIP stream.
There is no CPU fallback: if the library is missing, importing this package fails.

Public names mirror the C ABI of ``include/specconv.h``:
``sc_causal_conv_f32``, ``sc_causal_conv_bf16``, ``sc_causal_conv_ntt_i32``, their
``_ws`` variants, ``sc_causal_conv_ex``, ``sc_workspace_bytes``, ``sc_ntt_range_ok``,
``sc_status_string``, ``sc_version``, ``sc_prepare``, ``sc_causal_conv_noalloc`` (no
allocation: a static device scratch), and the gradient calls ``sc_causal_conv_bwd_f32``,
``sc_causal_conv_bwd_bf16``, ``sc_causal_conv_bwd_ntt_i32``, ``sc_causal_conv_bwd_ex``; plus
:func:`causal_conv` and :func:`causal_conv_bwd`, which dispatch on dtype; the exactly causal
real-valued calls ``sc_causal_conv_fixed_f32``, ``sc_causal_conv_fixed_f32_ws``,
``sc_fixed_range_ok`` and :func:`causal_conv_fixed`; and for a filter shared by the batch
``sc_filter_spectrum_bytes``, ``sc_filter_spectrum_{f32,bf16}``, ``sc_causal_conv_spec_{f32,bf16}``,
``sc_causal_conv_shared_{f32,bf16}`` with :func:`filter_spectrum`, :func:`causal_conv_spec`,
:func:`causal_conv_shared`.
"""
from __future__ import annotations

import ctypes
import os

import torch  # noqa: F401  -- load torch's HIP runtime first; libspecconv binds to it by soname

__all__ = [
    "SpecConvError", "lib", "causal_conv", "sc_causal_conv_f32", "sc_causal_conv_bf16",
    "sc_causal_conv_ntt_i32", "sc_causal_conv_f32_ws", "sc_causal_conv_bf16_ws",
    "sc_causal_conv_ntt_i32_ws", "sc_causal_conv_ex", "sc_workspace_bytes", "sc_ntt_range_ok",
    "sc_status_string", "sc_version", "sc_prepare", "sc_causal_conv_noalloc",
    "causal_conv_bwd", "sc_causal_conv_bwd_f32",
    "sc_causal_conv_bwd_bf16", "sc_causal_conv_bwd_ntt_i32", "sc_causal_conv_bwd_ex",
    "causal_conv_fixed", "sc_causal_conv_fixed_f32", "sc_causal_conv_fixed_f32_ws",
    "sc_fixed_range_ok", "filter_spectrum", "causal_conv_spec", "causal_conv_shared",
    "sc_filter_spectrum_bytes", "sc_filter_spectrum_f32", "sc_filter_spectrum_bf16",
    "sc_causal_conv_spec_f32", "sc_causal_conv_spec_bf16", "sc_causal_conv_shared_f32",
    "sc_causal_conv_shared_bf16", "causal_conv_spec_bwd", "causal_conv_shared_bwd",
    "sc_causal_conv_spec_bwd_f32", "sc_causal_conv_spec_bwd_bf16",
    "sc_causal_conv_shared_bwd_f32", "sc_causal_conv_shared_bwd_bf16", "causal_conv_blc",
    "sc_blc_workspace_bytes", "sc_causal_conv_blc_f32", "sc_causal_conv_blc_bf16",
    "sc_causal_conv_blc_ex", "gate", "gate_conv", "gate_conv_blc", "sc_gate_f32", "sc_gate_bf16",
    "sc_gate_conv_workspace_bytes", "sc_gate_conv_blc_workspace_bytes", "sc_gate_conv_ex",
    "sc_gate_conv_blc_ex", "sc_gate_conv_blc_f32", "sc_gate_conv_blc_bf16", "KIND_F32", "KIND_BF16", "KIND_NTT_I32", "KIND_FIXED_F32", "PATH_AUTO", "PATH_FUSED", "PATH_FOUR_STEP",
    "PATH_DIRECT", "PATH_NTT_MFMA", "PATH_FUSED_MFMA", "LIB_PATH",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libspecconv.so")

SC_OK, SC_ERR_INVALID_ARGUMENT, SC_ERR_UNSUPPORTED, SC_ERR_HIP, SC_ERR_WORKSPACE = range(5)
KIND_F32, KIND_BF16, KIND_NTT_I32, KIND_FIXED_F32 = 0, 1, 2, 3
PATH_AUTO, PATH_FUSED, PATH_FOUR_STEP, PATH_DIRECT, PATH_NTT_MFMA, PATH_FUSED_MFMA = 0, 1, 2, 3, 4, 5


class SpecConvError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__("%s: %s" % (what, sc_status_string(status)))
        self.status = status


class sc_options(ctypes.Structure):
    _fields_ = [("path", ctypes.c_int32), ("head", ctypes.c_int32),
                ("frac_v", ctypes.c_int32), ("frac_g", ctypes.c_int32),
                ("reserved", ctypes.c_int32 * 4)]


def _open():
    if not os.path.exists(LIB_PATH):
        raise ImportError("libspecconv.so is not built (run: python -m fft_causal_long_amd.build)")
    h = ctypes.CDLL(LIB_PATH)
    vp, i64, sz, st = ctypes.c_void_p, ctypes.c_int64, ctypes.c_size_t, ctypes.c_int
    for name in ("sc_causal_conv_f32", "sc_causal_conv_bf16", "sc_causal_conv_ntt_i32"):
        f = getattr(h, name)
        f.argtypes = [vp, vp, vp, i64, i64, i64, vp]
        f.restype = st
    for name in ("sc_causal_conv_f32_ws", "sc_causal_conv_bf16_ws", "sc_causal_conv_ntt_i32_ws"):
        f = getattr(h, name)
        f.argtypes = [vp, vp, vp, i64, i64, i64, vp, sz, vp]
        f.restype = st
    h.sc_causal_conv_ex.argtypes = [st, vp, vp, vp, i64, i64, i64,
                                    ctypes.POINTER(sc_options), vp, sz, vp]
    h.sc_causal_conv_ex.restype = st
    h.sc_blc_workspace_bytes.argtypes = [st, i64, i64, i64]
    h.sc_blc_workspace_bytes.restype = sz
    for name in ("sc_causal_conv_blc_f32", "sc_causal_conv_blc_bf16"):
        f = getattr(h, name)
        f.argtypes = [vp, vp, vp, i64, i64, i64, vp]
        f.restype = st
    h.sc_causal_conv_blc_ex.argtypes = [st, vp, vp, vp, i64, i64, i64,
                                        ctypes.POINTER(sc_options), vp, sz, vp]
    h.sc_causal_conv_blc_ex.restype = st
    for name in ("sc_gate_f32", "sc_gate_bf16"):
        f = getattr(h, name)
        f.argtypes = [vp, vp, vp, i64, i64, i64, vp]
        f.restype = st
    for name in ("sc_gate_conv_workspace_bytes", "sc_gate_conv_blc_workspace_bytes"):
        f = getattr(h, name)
        f.argtypes = [st, i64, i64, i64]
        f.restype = sz
    for name in ("sc_gate_conv_ex", "sc_gate_conv_blc_ex"):
        f = getattr(h, name)
        f.argtypes = [st, vp, vp, vp, vp, i64, i64, i64, ctypes.POINTER(sc_options), vp, sz, vp]
        f.restype = st
    for name in ("sc_gate_conv_blc_f32", "sc_gate_conv_blc_bf16"):
        f = getattr(h, name)
        f.argtypes = [vp, vp, vp, vp, i64, i64, i64, vp]
        f.restype = st
    for name in ("sc_causal_conv_bwd_f32", "sc_causal_conv_bwd_bf16", "sc_causal_conv_bwd_ntt_i32"):
        f = getattr(h, name)
        f.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, vp]
        f.restype = st
    h.sc_causal_conv_bwd_ex.argtypes = [st, vp, vp, vp, vp, vp, i64, i64, i64,
                                        ctypes.POINTER(sc_options), vp, sz, vp]
    h.sc_causal_conv_bwd_ex.restype = st
    h.sc_causal_conv_fixed_f32.argtypes = [vp, vp, vp, i64, i64, i64, ctypes.c_int32,
                                           ctypes.c_int32, vp]
    h.sc_causal_conv_fixed_f32.restype = st
    h.sc_causal_conv_fixed_f32_ws.argtypes = [vp, vp, vp, i64, i64, i64, ctypes.c_int32,
                                              ctypes.c_int32, vp, sz, vp]
    h.sc_causal_conv_fixed_f32_ws.restype = st
    h.sc_fixed_range_ok.argtypes = [ctypes.c_double, ctypes.c_double, ctypes.c_int32,
                                    ctypes.c_int32, i64]
    h.sc_fixed_range_ok.restype = ctypes.c_int
    h.sc_filter_spectrum_bytes.argtypes = [i64, i64]
    h.sc_filter_spectrum_bytes.restype = sz
    for name in ("sc_filter_spectrum_f32", "sc_filter_spectrum_bf16"):
        f = getattr(h, name)
        f.argtypes = [vp, vp, i64, i64, vp]
        f.restype = st
    for name in ("sc_causal_conv_spec_f32", "sc_causal_conv_spec_bf16",
                 "sc_causal_conv_shared_f32", "sc_causal_conv_shared_bf16"):
        f = getattr(h, name)
        f.argtypes = [vp, vp, vp, i64, i64, i64, vp]
        f.restype = st
    for name in ("sc_causal_conv_spec_bwd_f32", "sc_causal_conv_spec_bwd_bf16",
                 "sc_causal_conv_shared_bwd_f32", "sc_causal_conv_shared_bwd_bf16"):
        f = getattr(h, name)
        f.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, vp]
        f.restype = st
    h.sc_workspace_bytes.argtypes = [st, i64, i64, i64]
    h.sc_workspace_bytes.restype = sz
    h.sc_ntt_range_ok.argtypes = [i64, i64, i64]
    h.sc_ntt_range_ok.restype = ctypes.c_int
    h.sc_status_string.argtypes = [st]
    h.sc_status_string.restype = ctypes.c_char_p
    h.sc_version.argtypes = []
    h.sc_version.restype = ctypes.c_int
    h.sc_prepare.argtypes = [st, i64]
    h.sc_prepare.restype = st
    h.sc_causal_conv_noalloc.argtypes = [st, vp, vp, vp, i64, i64, i64, vp]
    h.sc_causal_conv_noalloc.restype = st
    return h


_lib = _open()


def lib():
    """The ctypes handle of libspecconv.so (argtypes set)."""
    return _lib


# ---------------------------------------------------------------- raw C-ABI mirrors

def sc_causal_conv_f32(v, g, r, B, C, L, stream):
    return _lib.sc_causal_conv_f32(v, g, r, B, C, L, stream)


def sc_causal_conv_bf16(v, g, r, B, C, L, stream):
    return _lib.sc_causal_conv_bf16(v, g, r, B, C, L, stream)


def sc_causal_conv_ntt_i32(v, g, r, B, C, L, stream):
    return _lib.sc_causal_conv_ntt_i32(v, g, r, B, C, L, stream)


def sc_causal_conv_f32_ws(v, g, r, B, C, L, ws, ws_bytes, stream):
    return _lib.sc_causal_conv_f32_ws(v, g, r, B, C, L, ws, ws_bytes, stream)


def sc_causal_conv_bf16_ws(v, g, r, B, C, L, ws, ws_bytes, stream):
    return _lib.sc_causal_conv_bf16_ws(v, g, r, B, C, L, ws, ws_bytes, stream)


def sc_causal_conv_ntt_i32_ws(v, g, r, B, C, L, ws, ws_bytes, stream):
    return _lib.sc_causal_conv_ntt_i32_ws(v, g, r, B, C, L, ws, ws_bytes, stream)


def sc_causal_conv_ex(kind, v, g, r, B, C, L, opt, ws, ws_bytes, stream):
    return _lib.sc_causal_conv_ex(kind, v, g, r, B, C, L, opt, ws, ws_bytes, stream)


def sc_causal_conv_bwd_f32(dr, v, g, dv, dg, B, C, L, stream):
    return _lib.sc_causal_conv_bwd_f32(dr, v, g, dv, dg, B, C, L, stream)


def sc_causal_conv_bwd_bf16(dr, v, g, dv, dg, B, C, L, stream):
    return _lib.sc_causal_conv_bwd_bf16(dr, v, g, dv, dg, B, C, L, stream)


def sc_causal_conv_bwd_ntt_i32(dr, v, g, dv, dg, B, C, L, stream):
    return _lib.sc_causal_conv_bwd_ntt_i32(dr, v, g, dv, dg, B, C, L, stream)


def sc_causal_conv_bwd_ex(kind, dr, v, g, dv, dg, B, C, L, opt, ws, ws_bytes, stream):
    return _lib.sc_causal_conv_bwd_ex(kind, dr, v, g, dv, dg, B, C, L, opt, ws, ws_bytes, stream)


def sc_causal_conv_fixed_f32(v, g, r, B, C, L, frac_v, frac_g, stream):
    return _lib.sc_causal_conv_fixed_f32(v, g, r, B, C, L, frac_v, frac_g, stream)


def sc_causal_conv_fixed_f32_ws(v, g, r, B, C, L, frac_v, frac_g, ws, ws_bytes, stream):
    return _lib.sc_causal_conv_fixed_f32_ws(v, g, r, B, C, L, frac_v, frac_g, ws, ws_bytes,
                                            stream)


def sc_fixed_range_ok(max_abs_v, max_abs_g, frac_v, frac_g, L) -> bool:
    return bool(_lib.sc_fixed_range_ok(float(max_abs_v), float(max_abs_g), int(frac_v),
                                       int(frac_g), int(L)))


def sc_filter_spectrum_bytes(C, L) -> int:
    return int(_lib.sc_filter_spectrum_bytes(C, L))


def sc_filter_spectrum_f32(k, spec, C, L, stream):
    return _lib.sc_filter_spectrum_f32(k, spec, C, L, stream)


def sc_filter_spectrum_bf16(k, spec, C, L, stream):
    return _lib.sc_filter_spectrum_bf16(k, spec, C, L, stream)


def sc_causal_conv_spec_f32(v, spec, r, B, C, L, stream):
    return _lib.sc_causal_conv_spec_f32(v, spec, r, B, C, L, stream)


def sc_causal_conv_spec_bf16(v, spec, r, B, C, L, stream):
    return _lib.sc_causal_conv_spec_bf16(v, spec, r, B, C, L, stream)


def sc_causal_conv_shared_f32(v, k, r, B, C, L, stream):
    return _lib.sc_causal_conv_shared_f32(v, k, r, B, C, L, stream)


def sc_causal_conv_shared_bf16(v, k, r, B, C, L, stream):
    return _lib.sc_causal_conv_shared_bf16(v, k, r, B, C, L, stream)


def sc_causal_conv_spec_bwd_f32(dr, v, spec, dv, dk, B, C, L, stream):
    return _lib.sc_causal_conv_spec_bwd_f32(dr, v, spec, dv, dk, B, C, L, stream)


def sc_causal_conv_spec_bwd_bf16(dr, v, spec, dv, dk, B, C, L, stream):
    return _lib.sc_causal_conv_spec_bwd_bf16(dr, v, spec, dv, dk, B, C, L, stream)


def sc_causal_conv_shared_bwd_f32(dr, v, k, dv, dk, B, C, L, stream):
    return _lib.sc_causal_conv_shared_bwd_f32(dr, v, k, dv, dk, B, C, L, stream)


def sc_causal_conv_shared_bwd_bf16(dr, v, k, dv, dk, B, C, L, stream):
    return _lib.sc_causal_conv_shared_bwd_bf16(dr, v, k, dv, dk, B, C, L, stream)


def sc_blc_workspace_bytes(kind, B, L, C) -> int:
    return int(_lib.sc_blc_workspace_bytes(kind, B, L, C))


def sc_causal_conv_blc_f32(v, g, r, B, L, C, stream):
    return _lib.sc_causal_conv_blc_f32(v, g, r, B, L, C, stream)


def sc_causal_conv_blc_bf16(v, g, r, B, L, C, stream):
    return _lib.sc_causal_conv_blc_bf16(v, g, r, B, L, C, stream)


def sc_causal_conv_blc_ex(kind, v, g, r, B, L, C, opt, ws, ws_bytes, stream):
    return _lib.sc_causal_conv_blc_ex(kind, v, g, r, B, L, C, opt, ws, ws_bytes, stream)


def sc_gate_f32(s, W, g, B, C, L, stream):
    return _lib.sc_gate_f32(s, W, g, B, C, L, stream)


def sc_gate_bf16(s, W, g, B, C, L, stream):
    return _lib.sc_gate_bf16(s, W, g, B, C, L, stream)


def sc_gate_conv_workspace_bytes(kind, B, C, L) -> int:
    return int(_lib.sc_gate_conv_workspace_bytes(kind, B, C, L))


def sc_gate_conv_blc_workspace_bytes(kind, B, L, C) -> int:
    return int(_lib.sc_gate_conv_blc_workspace_bytes(kind, B, L, C))


def sc_gate_conv_ex(kind, v, s, W, r, B, C, L, opt, ws, ws_bytes, stream):
    return _lib.sc_gate_conv_ex(kind, v, s, W, r, B, C, L, opt, ws, ws_bytes, stream)


def sc_gate_conv_blc_ex(kind, v, s, W, r, B, L, C, opt, ws, ws_bytes, stream):
    return _lib.sc_gate_conv_blc_ex(kind, v, s, W, r, B, L, C, opt, ws, ws_bytes, stream)


def sc_gate_conv_blc_f32(v, s, W, r, B, L, C, stream):
    return _lib.sc_gate_conv_blc_f32(v, s, W, r, B, L, C, stream)


def sc_gate_conv_blc_bf16(v, s, W, r, B, L, C, stream):
    return _lib.sc_gate_conv_blc_bf16(v, s, W, r, B, L, C, stream)


def sc_workspace_bytes(kind, B, C, L) -> int:
    return int(_lib.sc_workspace_bytes(kind, B, C, L))


def sc_ntt_range_ok(max_abs_v, max_abs_g, L) -> bool:
    return bool(_lib.sc_ntt_range_ok(max_abs_v, max_abs_g, L))


def sc_status_string(status: int) -> str:
    return _lib.sc_status_string(int(status)).decode()


def sc_version() -> int:
    return int(_lib.sc_version())


def sc_prepare(kind, L):
    return _lib.sc_prepare(kind, L)


def sc_causal_conv_noalloc(kind, v, g, r, B, C, L, stream):
    return _lib.sc_causal_conv_noalloc(kind, v, g, r, B, C, L, stream)


# ---------------------------------------------------------------- tensor front end

_KIND_OF_DTYPE = {torch.float32: KIND_F32, torch.bfloat16: KIND_BF16, torch.int32: KIND_NTT_I32}


def _shape3(t: torch.Tensor):
    if t.dim() == 3:
        return tuple(int(x) for x in t.shape)
    if t.dim() == 0:
        raise ValueError("causal_conv needs at least 1 dimension")
    L = int(t.shape[-1])
    lead = 1
    for s in t.shape[:-1]:
        lead *= int(s)
    return lead, 1, L


def causal_conv(v: torch.Tensor, g: torch.Tensor, out: torch.Tensor | None = None, *,
                path: int | None = None, head: int | None = None,
                workspace: torch.Tensor | None = None) -> torch.Tensor:
    """r = causal_conv(v, g) along the last axis, on v's device and torch's current stream.

    dtype selects the kind: float32 -> sc_causal_conv_f32, bfloat16 -> sc_causal_conv_bf16,
    int32 -> sc_causal_conv_ntt_i32 (exact mod p).  v, g (and out) must be contiguous
    device tensors of one shape and dtype.  ``path``/``head`` go through
    sc_causal_conv_ex; ``workspace`` is an optional caller-owned uint8 device tensor."""
    if v.shape != g.shape or v.dtype != g.dtype:
        raise ValueError("v and g must have the same shape and dtype")
    if v.dtype not in _KIND_OF_DTYPE:
        raise TypeError("unsupported dtype %s" % v.dtype)
    if not (v.is_cuda and g.is_cuda) or v.device != g.device:
        raise ValueError("v and g must be on the same GPU")
    if not (v.is_contiguous() and g.is_contiguous()):
        raise ValueError("v and g must be contiguous")
    if out is None:
        out = torch.empty_like(v)
    elif out.shape != v.shape or out.dtype != v.dtype or out.device != v.device \
            or not out.is_contiguous():
        raise ValueError("out must match v in shape, dtype, device and be contiguous")
    B, C, L = _shape3(v)
    kind = _KIND_OF_DTYPE[v.dtype]
    ws_ptr, ws_bytes = None, 0
    if workspace is not None:
        if not workspace.is_cuda or workspace.device != v.device or not workspace.is_contiguous():
            raise ValueError("workspace must be a contiguous tensor on v's device")
        ws_ptr, ws_bytes = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    with torch.cuda.device(v.device):
        stream = torch.cuda.current_stream(v.device).cuda_stream
        if path is None and head is None:
            if ws_ptr is None:
                fn = (_lib.sc_causal_conv_f32, _lib.sc_causal_conv_bf16,
                      _lib.sc_causal_conv_ntt_i32)[kind]
                st = fn(v.data_ptr(), g.data_ptr(), out.data_ptr(), B, C, L, stream)
            else:
                fn = (_lib.sc_causal_conv_f32_ws, _lib.sc_causal_conv_bf16_ws,
                      _lib.sc_causal_conv_ntt_i32_ws)[kind]
                st = fn(v.data_ptr(), g.data_ptr(), out.data_ptr(), B, C, L, ws_ptr, ws_bytes,
                        stream)
        else:
            opt = sc_options(PATH_AUTO if path is None else int(path),
                             -1 if head is None else int(head))
            st = _lib.sc_causal_conv_ex(kind, v.data_ptr(), g.data_ptr(), out.data_ptr(),
                                        B, C, L, ctypes.byref(opt), ws_ptr, ws_bytes, stream)
    if st != SC_OK:
        raise SpecConvError(st, "causal_conv")
    return out


def causal_conv_blc(v: torch.Tensor, g: torch.Tensor, out: torch.Tensor | None = None, *,
                    path: int | None = None, head: int | None = None,
                    workspace: torch.Tensor | None = None) -> torch.Tensor:
    """r[..., t, c] = sum_{j<=t} v[..., j, c] g[..., t-j, c]: the causal convolution along the
    second-to-last axis of token-major (..., L, C) tensors (sc_causal_conv_blc_ex).  Kinds as
    :func:`causal_conv` (float32, bfloat16, int32 exact); ``workspace`` optional, at least
    sc_blc_workspace_bytes(kind, B, L, C) bytes."""
    if v.shape != g.shape or v.dtype != g.dtype:
        raise ValueError("v and g must have the same shape and dtype")
    if v.dtype not in _KIND_OF_DTYPE:
        raise TypeError("unsupported dtype %s" % v.dtype)
    if not (v.is_cuda and g.is_cuda) or v.device != g.device:
        raise ValueError("v and g must be on the same GPU")
    if not (v.is_contiguous() and g.is_contiguous()):
        raise ValueError("v and g must be contiguous")
    if v.dim() < 2:
        raise ValueError("v must be (..., L, C)")
    out = _out_like(v, out, "out")
    L, C = int(v.shape[-2]), int(v.shape[-1])
    B = 1
    for s_ in v.shape[:-2]:
        B *= int(s_)
    kind = _KIND_OF_DTYPE[v.dtype]
    ws_ptr, ws_bytes = None, 0
    if workspace is not None:
        if not workspace.is_cuda or workspace.device != v.device or not workspace.is_contiguous():
            raise ValueError("workspace must be a contiguous tensor on v's device")
        ws_ptr, ws_bytes = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    opt = sc_options(PATH_AUTO if path is None else int(path), -1 if head is None else int(head))
    with torch.cuda.device(v.device):
        stream = torch.cuda.current_stream(v.device).cuda_stream
        st = _lib.sc_causal_conv_blc_ex(kind, v.data_ptr(), g.data_ptr(), out.data_ptr(), B, L,
                                        C, ctypes.byref(opt), ws_ptr, ws_bytes, stream)
    if st != SC_OK:
        raise SpecConvError(st, "causal_conv_blc")
    return out


def _out_like(x: torch.Tensor, out: torch.Tensor | None, name: str) -> torch.Tensor:
    if out is None:
        return torch.empty_like(x)
    if out.shape != x.shape or out.dtype != x.dtype or out.device != x.device \
            or not out.is_contiguous():
        raise ValueError("%s must match the inputs in shape, dtype, device and be contiguous"
                         % name)
    return out


def causal_conv_bwd(dr: torch.Tensor, v: torch.Tensor, g: torch.Tensor,
                    dv: torch.Tensor | None = None, dg: torch.Tensor | None = None, *,
                    path: int | None = None, head: int | None = None,
                    workspace: torch.Tensor | None = None):
    """Gradients of sum(dr * causal_conv(v, g)) along the last axis: returns (dv, dg) with
    dv[..., j] = sum_{t>=j} dr[..., t] g[..., t-j] and dg[..., k] = sum_{t>=k} dr[..., t]
    v[..., t-k].  Same dtype rules, devices, stream and options as :func:`causal_conv`."""
    if not (dr.shape == v.shape == g.shape) or not (dr.dtype == v.dtype == g.dtype):
        raise ValueError("dr, v and g must have the same shape and dtype")
    if v.dtype not in _KIND_OF_DTYPE:
        raise TypeError("unsupported dtype %s" % v.dtype)
    if not (dr.is_cuda and v.is_cuda and g.is_cuda) or not (dr.device == v.device == g.device):
        raise ValueError("dr, v and g must be on the same GPU")
    if not (dr.is_contiguous() and v.is_contiguous() and g.is_contiguous()):
        raise ValueError("dr, v and g must be contiguous")
    dv = _out_like(v, dv, "dv")
    dg = _out_like(v, dg, "dg")
    B, C, L = _shape3(v)
    kind = _KIND_OF_DTYPE[v.dtype]
    ws_ptr, ws_bytes = None, 0
    if workspace is not None:
        if not workspace.is_cuda or workspace.device != v.device or not workspace.is_contiguous():
            raise ValueError("workspace must be a contiguous tensor on v's device")
        ws_ptr, ws_bytes = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    ptrs = (dr.data_ptr(), v.data_ptr(), g.data_ptr(), dv.data_ptr(), dg.data_ptr())
    with torch.cuda.device(v.device):
        stream = torch.cuda.current_stream(v.device).cuda_stream
        if path is None and head is None and ws_ptr is None:
            fn = (_lib.sc_causal_conv_bwd_f32, _lib.sc_causal_conv_bwd_bf16,
                  _lib.sc_causal_conv_bwd_ntt_i32)[kind]
            st = fn(*ptrs, B, C, L, stream)
        else:
            opt = sc_options(PATH_AUTO if path is None else int(path),
                             -1 if head is None else int(head))
            st = _lib.sc_causal_conv_bwd_ex(kind, *ptrs, B, C, L, ctypes.byref(opt), ws_ptr,
                                            ws_bytes, stream)
    if st != SC_OK:
        raise SpecConvError(st, "causal_conv_bwd")
    return dv, dg


def causal_conv_fixed(v: torch.Tensor, g: torch.Tensor, frac_v: int, frac_g: int,
                      out: torch.Tensor | None = None, *,
                      workspace: torch.Tensor | None = None) -> torch.Tensor:
    """Exactly causal float32 convolution on fixed-point encodings (sc_causal_conv_fixed_f32):
    r_t = round_f32(sum_{j<=t} round(v_j 2^frac_v) round(g_{t-j} 2^frac_g) 2^-(frac_v+frac_g))
    along the last axis.  v, g: contiguous float32 tensors on one GPU."""
    if v.shape != g.shape or v.dtype != torch.float32 or g.dtype != torch.float32:
        raise ValueError("v and g must be float32 tensors of one shape")
    if not (v.is_cuda and g.is_cuda) or v.device != g.device:
        raise ValueError("v and g must be on the same GPU")
    if not (v.is_contiguous() and g.is_contiguous()):
        raise ValueError("v and g must be contiguous")
    out = _out_like(v, out, "out")
    B, C, L = _shape3(v)
    with torch.cuda.device(v.device):
        stream = torch.cuda.current_stream(v.device).cuda_stream
        if workspace is None:
            st = _lib.sc_causal_conv_fixed_f32(v.data_ptr(), g.data_ptr(), out.data_ptr(), B, C,
                                               L, int(frac_v), int(frac_g), stream)
        else:
            if not workspace.is_cuda or workspace.device != v.device or \
                    not workspace.is_contiguous():
                raise ValueError("workspace must be a contiguous tensor on v's device")
            st = _lib.sc_causal_conv_fixed_f32_ws(
                v.data_ptr(), g.data_ptr(), out.data_ptr(), B, C, L, int(frac_v), int(frac_g),
                workspace.data_ptr(), workspace.numel() * workspace.element_size(), stream)
    if st != SC_OK:
        raise SpecConvError(st, "causal_conv_fixed")
    return out


def _bcl(v: torch.Tensor, k: torch.Tensor):
    """(B, C, L) of v for a filter k of shape (C, L): v is (..., C, L)."""
    if k.dim() != 2 or v.dim() < 2 or tuple(v.shape[-2:]) != tuple(k.shape):
        raise ValueError("k must be (C, L) and v (..., C, L)")
    C, L = int(k.shape[0]), int(k.shape[1])
    B = 1
    for s_ in v.shape[:-2]:
        B *= int(s_)
    return B, C, L


_SPEC_FN = {torch.float32: ("sc_filter_spectrum_f32", "sc_causal_conv_spec_f32",
                            "sc_causal_conv_shared_f32"),
            torch.bfloat16: ("sc_filter_spectrum_bf16", "sc_causal_conv_spec_bf16",
                             "sc_causal_conv_shared_bf16")}


def _check_float(*ts):
    for t in ts:
        if t.dtype not in _SPEC_FN:
            raise TypeError("filter calls take float32 or bfloat16 tensors")
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError("tensors must be contiguous and on the GPU")
    if len({t.dtype for t in ts}) != 1 or len({t.device for t in ts}) != 1:
        raise ValueError("tensors must share dtype and device")


def filter_spectrum(k: torch.Tensor) -> torch.Tensor:
    """Spectrum of the filters k (C, L), float32 or bfloat16, as an opaque uint8 device tensor
    for :func:`causal_conv_spec` (sc_filter_spectrum_*)."""
    _check_float(k)
    if k.dim() != 2:
        raise ValueError("k must be (C, L)")
    C, L = int(k.shape[0]), int(k.shape[1])
    nbytes = sc_filter_spectrum_bytes(C, L)
    if nbytes == 0 and C > 0:
        raise SpecConvError(SC_ERR_UNSUPPORTED, "filter_spectrum")
    spec = torch.empty(max(nbytes, 8), dtype=torch.uint8, device=k.device)
    with torch.cuda.device(k.device):
        stream = torch.cuda.current_stream(k.device).cuda_stream
        st = getattr(_lib, _SPEC_FN[k.dtype][0])(k.data_ptr(), spec.data_ptr(), C, L, stream)
    if st != SC_OK:
        raise SpecConvError(st, "filter_spectrum")
    spec.sc_shape = (C, L, k.dtype)
    return spec


def causal_conv_spec(v: torch.Tensor, spec: torch.Tensor, C: int, L: int,
                     out: torch.Tensor | None = None) -> torch.Tensor:
    """r[b, c, t] = sum_{j<=t} v[b, c, j] k[c, t-j] from the spectrum of k (made by
    :func:`filter_spectrum` for this C and L); v is (..., C, L)."""
    _check_float(v)
    if tuple(v.shape[-2:]) != (C, L):
        raise ValueError("v must be (..., C, L)")
    if spec.dtype != torch.uint8 or spec.device != v.device or \
            spec.numel() < sc_filter_spectrum_bytes(C, L):
        raise ValueError("spec must be a spectrum tensor of this C and L on v's device")
    out = _out_like(v, out, "out")
    B = v.numel() // max(C * L, 1)
    with torch.cuda.device(v.device):
        stream = torch.cuda.current_stream(v.device).cuda_stream
        st = getattr(_lib, _SPEC_FN[v.dtype][1])(v.data_ptr(), spec.data_ptr(), out.data_ptr(),
                                                 B, C, L, stream)
    if st != SC_OK:
        raise SpecConvError(st, "causal_conv_spec")
    return out


def causal_conv_shared(v: torch.Tensor, k: torch.Tensor,
                       out: torch.Tensor | None = None) -> torch.Tensor:
    """r[b, c, t] = sum_{j<=t} v[b, c, j] k[c, t-j] with one filter per channel shared by the
    batch (sc_causal_conv_shared_*); v is (..., C, L), k is (C, L)."""
    _check_float(v, k)
    B, C, L = _bcl(v, k)
    out = _out_like(v, out, "out")
    with torch.cuda.device(v.device):
        stream = torch.cuda.current_stream(v.device).cuda_stream
        st = getattr(_lib, _SPEC_FN[v.dtype][2])(v.data_ptr(), k.data_ptr(), out.data_ptr(), B,
                                                 C, L, stream)
    if st != SC_OK:
        raise SpecConvError(st, "causal_conv_shared")
    return out


_BWD_FN = {torch.float32: ("sc_causal_conv_spec_bwd_f32", "sc_causal_conv_shared_bwd_f32"),
           torch.bfloat16: ("sc_causal_conv_spec_bwd_bf16", "sc_causal_conv_shared_bwd_bf16")}


def _filter_grad_like(v: torch.Tensor, C: int, L: int, dk: torch.Tensor | None) -> torch.Tensor:
    if dk is None:
        return torch.empty((C, L), dtype=v.dtype, device=v.device)
    if dk.dtype != v.dtype or dk.device != v.device or tuple(dk.shape) != (C, L) or \
            not dk.is_contiguous():
        raise ValueError("dk must be a contiguous (C, L) tensor of v's dtype and device")
    return dk


def causal_conv_spec_bwd(dr: torch.Tensor, v: torch.Tensor, spec: torch.Tensor, C: int, L: int,
                         dv: torch.Tensor | None = None, dk: torch.Tensor | None = None):
    """(dv, dk) of r = causal_conv_spec(v, spec) for the output gradient dr, with dk summed over
    the batch (sc_causal_conv_spec_bwd_*); spec from :func:`filter_spectrum` for this C, L."""
    _check_float(dr, v)
    if tuple(v.shape[-2:]) != (C, L) or dr.shape != v.shape:
        raise ValueError("dr and v must be (..., C, L) of one shape")
    if spec.dtype != torch.uint8 or spec.device != v.device or \
            spec.numel() < sc_filter_spectrum_bytes(C, L):
        raise ValueError("spec must be a spectrum tensor of this C and L on v's device")
    dv = _out_like(v, dv, "dv")
    dk = _filter_grad_like(v, C, L, dk)
    B = v.numel() // max(C * L, 1)
    with torch.cuda.device(v.device):
        stream = torch.cuda.current_stream(v.device).cuda_stream
        st = getattr(_lib, _BWD_FN[v.dtype][0])(dr.data_ptr(), v.data_ptr(), spec.data_ptr(),
                                                dv.data_ptr(), dk.data_ptr(), B, C, L, stream)
    if st != SC_OK:
        raise SpecConvError(st, "causal_conv_spec_bwd")
    return dv, dk


def causal_conv_shared_bwd(dr: torch.Tensor, v: torch.Tensor, k: torch.Tensor,
                           dv: torch.Tensor | None = None, dk: torch.Tensor | None = None):
    """(dv, dk) of r = causal_conv_shared(v, k) for the output gradient dr, with dk summed over
    the batch (sc_causal_conv_shared_bwd_*)."""
    _check_float(dr, v, k)
    B, C, L = _bcl(v, k)
    if dr.shape != v.shape:
        raise ValueError("dr must have v's shape")
    dv = _out_like(v, dv, "dv")
    dk = _filter_grad_like(v, C, L, dk)
    with torch.cuda.device(v.device):
        stream = torch.cuda.current_stream(v.device).cuda_stream
        st = getattr(_lib, _BWD_FN[v.dtype][1])(dr.data_ptr(), v.data_ptr(), k.data_ptr(),
                                                dv.data_ptr(), dk.data_ptr(), B, C, L, stream)
    if st != SC_OK:
        raise SpecConvError(st, "causal_conv_shared_bwd")
    return dv, dk


def _gate_args(s: torch.Tensor, W: torch.Tensor, *others: torch.Tensor):
    for t in (s, W) + others:
        if t.dtype not in (torch.float32, torch.bfloat16):
            raise TypeError("gate calls take float32 or bfloat16 tensors")
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError("tensors must be contiguous and on the GPU")
    if len({t.dtype for t in (s, W) + others}) != 1 or \
            len({t.device for t in (s, W) + others}) != 1:
        raise ValueError("tensors must share dtype and device")
    if W.dim() != 3 or W.shape[1] != 64 or W.shape[2] != 3:
        raise ValueError("W must be (C, 64, 3)")
    return KIND_F32 if s.dtype == torch.float32 else KIND_BF16


def _ws_args(workspace, dev):
    if workspace is None:
        return None, 0
    if not workspace.is_cuda or workspace.device != dev or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous tensor on the inputs' device")
    return workspace.data_ptr(), workspace.numel() * workspace.element_size()


def gate(s: torch.Tensor, W: torch.Tensor, out: torch.Tensor | None = None) -> torch.Tensor:
    """g = Conv1d_G2(sigmoid(s)) (sc_gate_*): s (..., C, L) channel-major, W (C, 64, 3)."""
    kind = _gate_args(s, W)
    if s.dim() < 2 or s.shape[-2] != W.shape[0]:
        raise ValueError("s must be (..., C, L) with C = W.shape[0]")
    C, L = int(s.shape[-2]), int(s.shape[-1])
    B = s.numel() // max(C * L, 1)
    out = _out_like(s, out, "out")
    fn = _lib.sc_gate_f32 if kind == KIND_F32 else _lib.sc_gate_bf16
    with torch.cuda.device(s.device):
        stream = torch.cuda.current_stream(s.device).cuda_stream
        st = fn(s.data_ptr(), W.data_ptr(), out.data_ptr(), B, C, L, stream)
    if st != SC_OK:
        raise SpecConvError(st, "gate")
    return out


def gate_conv(v: torch.Tensor, s: torch.Tensor, W: torch.Tensor, out: torch.Tensor | None = None,
              *, path: int | None = None, head: int | None = None,
              workspace: torch.Tensor | None = None) -> torch.Tensor:
    """r = causal_conv(v, gate(s, W)) with v, s (..., C, L) channel-major (sc_gate_conv_ex)."""
    kind = _gate_args(s, W, v)
    if v.shape != s.shape or v.dim() < 2 or v.shape[-2] != W.shape[0]:
        raise ValueError("v and s must be (..., C, L) of one shape, C = W.shape[0]")
    C, L = int(v.shape[-2]), int(v.shape[-1])
    B = v.numel() // max(C * L, 1)
    out = _out_like(v, out, "out")
    ws_ptr, ws_bytes = _ws_args(workspace, v.device)
    opt = sc_options(PATH_AUTO if path is None else int(path), -1 if head is None else int(head))
    with torch.cuda.device(v.device):
        stream = torch.cuda.current_stream(v.device).cuda_stream
        st = _lib.sc_gate_conv_ex(kind, v.data_ptr(), s.data_ptr(), W.data_ptr(), out.data_ptr(),
                                  B, C, L, ctypes.byref(opt), ws_ptr, ws_bytes, stream)
    if st != SC_OK:
        raise SpecConvError(st, "gate_conv")
    return out


def gate_conv_blc(v: torch.Tensor, s: torch.Tensor, W: torch.Tensor,
                  out: torch.Tensor | None = None, *, path: int | None = None,
                  head: int | None = None, workspace: torch.Tensor | None = None) -> torch.Tensor:
    """r = causal_conv(v, gate(s, W)) along the token axis of token-major (..., L, C) tensors
    (sc_gate_conv_blc_ex)."""
    kind = _gate_args(s, W, v)
    if v.shape != s.shape or v.dim() < 2 or v.shape[-1] != W.shape[0]:
        raise ValueError("v and s must be (..., L, C) of one shape, C = W.shape[0]")
    L, C = int(v.shape[-2]), int(v.shape[-1])
    B = v.numel() // max(C * L, 1)
    out = _out_like(v, out, "out")
    ws_ptr, ws_bytes = _ws_args(workspace, v.device)
    opt = sc_options(PATH_AUTO if path is None else int(path), -1 if head is None else int(head))
    with torch.cuda.device(v.device):
        stream = torch.cuda.current_stream(v.device).cuda_stream
        st = _lib.sc_gate_conv_blc_ex(kind, v.data_ptr(), s.data_ptr(), W.data_ptr(),
                                      out.data_ptr(), B, L, C, ctypes.byref(opt), ws_ptr,
                                      ws_bytes, stream)
    if st != SC_OK:
        raise SpecConvError(st, "gate_conv_blc")
    return out
