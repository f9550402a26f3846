"""Thin ctypes binding of libwoq (include/woq.h).

Every function named ``woq_*`` here marshals its arguments and calls the C
entry point of the same name; nothing is computed in Python.  Host arrays are
NumPy arrays; device buffers are torch tensors (torch is used only for device
memory and streams).  Errors raise :class:`WoqError`.  The library must have
been built (``python -m weight_only_quantized_quantize_amd.build``); there is
no fallback.
"""
from __future__ import annotations

import ctypes
import os
import sys
from ctypes import POINTER, c_double, c_float, c_int, c_int32, c_int64, c_uint8, c_uint16, c_void_p

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libwoq.so")

WOQ_OK, WOQ_EINVAL, WOQ_EALIGN, WOQ_ENOMEM, WOQ_EHIP, WOQ_EUNSUPPORTED, WOQ_ERANGE = 0, -1, -2, -3, -4, -5, -6
WOQ_EIO, WOQ_EFORMAT = -8, -9
MAX_SEGMENTS = 8


class WoqError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = _lib().woq_strerror(status).decode() if _LIB is not None else str(status)
        if status == WOQ_EHIP and _LIB is not None:
            msg += f" (hipError {_LIB.woq_last_hip_error()})"
        super().__init__(f"{where}: {msg} [{status}]")


class Int4oGeom(ctypes.Structure):
    _fields_ = [(n, c_int64) for n in ("K", "n_out", "K_bg", "G", "K_pad", "G4", "n_out8", "xp_len")]

    def as_dict(self):
        return {n: int(getattr(self, n)) for n, _ in self._fields_}


class Int8W(ctypes.Structure):
    _fields_ = [("codes", c_void_p), ("N", c_int64), ("K", c_int64), ("nseg", c_int32),
                ("seg_end", c_int64 * MAX_SEGMENTS), ("seg_scale", c_float * MAX_SEGMENTS)]


class Int4oW(ctypes.Structure):
    _fields_ = [("codes", c_void_p), ("scales", c_void_p), ("w_out", c_void_p), ("N", c_int64),
                ("geom", Int4oGeom)]


class StackStep(ctypes.Structure):
    _fields_ = [("fmt", c_int32), ("in_slot", c_int32), ("out_slot", c_int32), ("w8", Int8W), ("w4", Int4oW),
                ("perm", c_void_p)]


class PagerStep(ctypes.Structure):
    _fields_ = [("code_offset", c_int64), ("w", Int8W)]


FMT_INT8, FMT_INT4O = 1, 2

_LIB = None

_SIGS = {
    "woq_strerror": (ctypes.c_char_p, [c_int]),
    "woq_last_hip_error": (c_int, []),
    "woq_abi_version": (c_int, []),
    "woq_int4o_geometry": (c_int, [c_int64, c_int64, POINTER(Int4oGeom)]),
    "woq_quantize_int8": (c_int, [c_void_p, c_int64, c_int64, c_void_p, POINTER(c_float)]),
    "woq_colabs_accumulate": (c_int, [c_void_p, c_int64, c_int64, c_void_p]),
    "woq_outlier_select": (c_int, [c_void_p, c_void_p, c_int64, c_int64, c_int64, c_void_p]),
    "woq_outlier_perm": (c_int, [POINTER(c_void_p), POINTER(c_int64), c_int32, c_int64, c_void_p, c_int64, c_int64,
                                 c_void_p]),
    "woq_outlier_perm_sums": (c_int, [POINTER(c_void_p), c_int32, c_int64, c_void_p, c_int64, c_int64, c_void_p]),
    "woq_quantize_int4o": (c_int, [c_void_p, c_int64, c_int64, c_void_p, c_int64, c_void_p, c_void_p, c_void_p]),
    "woq_unpack_int4": (c_int, [c_void_p, c_int64, c_int64, c_void_p]),
    "woq_int8_dev_bytes": (c_int64, [c_int64, c_int64]),
    "woq_layout_int8": (c_int, [c_void_p, c_int64, c_int64, c_void_p]),
    "woq_layout_int8_inverse": (c_int, [c_void_p, c_int64, c_int64, c_void_p]),
    "woq_int4o_dev_sizes": (c_int, [c_int64, POINTER(Int4oGeom), POINTER(c_int64), POINTER(c_int64), POINTER(c_int64)]),
    "woq_layout_int4o": (c_int, [c_void_p, c_void_p, c_void_p, c_int64, POINTER(Int4oGeom), c_void_p, c_void_p, c_void_p]),
    "woq_layout_int4o_inverse": (c_int, [c_void_p, c_void_p, c_void_p, c_int64, POINTER(Int4oGeom), c_void_p, c_void_p, c_void_p]),
    "woq_permute_x": (c_int, [c_void_p, c_int64, c_void_p, c_int64, POINTER(Int4oGeom), c_void_p, c_void_p]),
    "woq_qgemv_int8": (c_int, [POINTER(Int8W), c_void_p, c_int64, c_int64, c_void_p, c_int64, c_void_p]),
    "woq_embed_int8": (c_int, [POINTER(Int8W), c_void_p, c_int64, c_void_p, c_int64, c_void_p]),
    "woq_qgemv_int4o": (c_int, [POINTER(Int4oW), c_void_p, c_int64, c_void_p, c_int64, c_void_p]),
    "woq_qgemm_int4o": (c_int, [POINTER(Int4oW), c_void_p, c_int64, c_void_p, c_int64, c_void_p]),
    "woq_perm_positions": (c_int, [c_void_p, POINTER(Int4oGeom), c_void_p]),
    "woq_stream_read": (c_int, [c_void_p, c_int64, c_void_p]),
    "woq_dispatch_floor": (c_int, [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, c_void_p,
                                   ctypes.POINTER(ctypes.c_float), ctypes.POINTER(ctypes.c_float)]),
    "woq_qgemv_int4o_x": (c_int, [POINTER(Int4oW), c_void_p, c_int64, c_void_p, c_int64, c_void_p, c_int64,
                                  c_void_p]),
    "woq_qgemv_int4o_x_supported": (c_int, [POINTER(Int4oGeom), c_int64]),
    "woq_qgemm_int4o_x": (c_int, [POINTER(Int4oW), c_void_p, c_int64, c_void_p, c_int64, c_void_p, c_int64,
                                  c_void_p]),
    "woq_qgemm_int4o_x_supported": (c_int, [POINTER(Int4oGeom), c_int64, c_int64]),
    "woq_stack_create": (c_int, [POINTER(StackStep), c_int32, c_int64, POINTER(c_void_p)]),
    "woq_stack_run": (c_int, [c_void_p, POINTER(c_void_p), POINTER(c_void_p), c_int64, c_void_p]),
    "woq_stack_launches": (c_int, [c_void_p, c_int64, POINTER(c_int32)]),
    "woq_stack_time": (c_int, [c_void_p, POINTER(c_void_p), POINTER(c_void_p), c_int64, c_void_p, c_int32,
                               POINTER(c_float), POINTER(c_float)]),
    "woq_stack_destroy": (c_int, [c_void_p]),
    "woq_quantize_int8_dev": (c_int, [c_void_p, c_int64, c_int64, c_void_p, c_void_p, c_void_p, c_void_p]),
    "woq_quantize_int4o_dev": (c_int, [c_void_p, c_int64, c_void_p, POINTER(Int4oGeom), c_void_p, c_void_p,
                                       c_void_p, c_void_p, c_void_p]),
    "woq_pool_save": (c_int, [ctypes.c_char_p, c_void_p, c_int64, POINTER(c_void_p), POINTER(c_int64), c_int32]),
    "woq_pool_info": (c_int, [ctypes.c_char_p, POINTER(c_int32), POINTER(c_int64), POINTER(c_int64), c_int32,
                              c_void_p, c_int64]),
    "woq_pool_read_block": (c_int, [ctypes.c_char_p, c_int32, c_void_p, c_int64]),
    "woq_qgemm_int4o_splitk": (c_int, [POINTER(Int4oW), c_void_p, c_int64, c_void_p, c_int64, c_int32, c_void_p,
                                       c_int64, c_void_p]),
    "woq_qgemm_int4o_splitk_workspace": (c_int64, [c_int64, c_int64, c_int32]),
    "woq_qgemm_int4o_splitk_noalloc": (c_int, [POINTER(Int4oW), c_void_p, c_int64, c_void_p, c_int64, c_int32,
                                               c_void_p]),
    "woq_plan_tiers": (c_int, [c_void_p, c_int32, c_int64, c_void_p, POINTER(c_int64)]),
    "woq_tiered_create": (c_int, [c_void_p, POINTER(c_int64), POINTER(c_int64), c_int32, POINTER(StackStep),
                                  c_int32, c_int64, POINTER(c_void_p)]),
    "woq_pager_create": (c_int, [c_void_p, POINTER(c_int64), POINTER(c_int64), c_int32, POINTER(PagerStep), c_int32,
                                 c_int64, POINTER(c_void_p)]),
    "woq_pager_run": (c_int, [c_void_p, POINTER(c_void_p), POINTER(c_void_p), c_int64, c_void_p, c_void_p]),
    "woq_pager_destroy": (c_int, [c_void_p]),
    "woq_pager_streamed_layers": (c_int, [c_void_p, POINTER(c_int32)]),
    "woq_pager_time": (c_int, [c_void_p, POINTER(c_void_p), POINTER(c_void_p), c_int64, c_void_p, c_void_p,
                               POINTER(c_float), POINTER(c_float), POINTER(c_float), POINTER(c_float)]),
}

# symbols the header declares (checked by the CPU tests)
EXPORTS = tuple(_SIGS)


def _lib():
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"libwoq.so is not built ({LIB_PATH}); run "
                               "`python -m weight_only_quantized_quantize_amd.build`")
        # torch ships its own HIP runtime: load it before the library, so that
        # the library binds to that runtime instead of loading a second one
        # (with two in one process the GPU was reported missing on MI355X)
        try:
            import torch  # noqa: F401
        except ImportError:
            pass
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _LIB = lib
    return _LIB


def lib():
    """The loaded ctypes library (loads it on first use)."""
    return _lib()


def require_gpu():
    """Raise unless a GPU is visible and the HIP library is loaded."""
    import torch
    if not torch.cuda.is_available():
        raise RuntimeError("no GPU visible: the weight-only quantised kernels run only on the GPU")
    _lib()


def _check(status: int, where: str):
    if status != WOQ_OK:
        raise WoqError(status, where)


def _ptr(a) -> int:
    """Address of a NumPy array (C-contiguous) or a torch tensor (contiguous)."""
    if a is None:
        return None
    if isinstance(a, np.ndarray):
        assert a.flags["C_CONTIGUOUS"], "array must be C-contiguous"
        return a.ctypes.data
    assert a.is_contiguous(), "tensor must be contiguous"
    return a.data_ptr()


def _stream(stream) -> int | None:
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    import torch
    return torch.cuda.current_stream().cuda_stream


# ----------------------------------------------------------------- geometry

def woq_int4o_geometry(K: int, n_out: int = -1) -> Int4oGeom:
    g = Int4oGeom()
    _check(_lib().woq_int4o_geometry(K, n_out, ctypes.byref(g)), "woq_int4o_geometry")
    return g


# ---------------------------------------------------------------- host prep

def woq_quantize_int8(W: np.ndarray):
    W = np.ascontiguousarray(W, np.float32)
    N, K = W.shape
    q = np.empty((N, K), np.int8)
    s = c_float()
    _check(_lib().woq_quantize_int8(_ptr(W), N, K, _ptr(q), ctypes.byref(s)), "woq_quantize_int8")
    return q, np.float32(s.value)


def woq_colabs_accumulate(W: np.ndarray, colsum: np.ndarray):
    W = np.ascontiguousarray(W, np.float32)
    assert colsum.dtype == np.float64 and colsum.shape == (W.shape[1],)
    _check(_lib().woq_colabs_accumulate(_ptr(W), W.shape[0], W.shape[1], _ptr(colsum)), "woq_colabs_accumulate")
    return colsum


def woq_outlier_select(colsum: np.ndarray, xprof: np.ndarray, n_out: int = -1) -> np.ndarray:
    colsum = np.ascontiguousarray(colsum, np.float64)
    xprof = np.ascontiguousarray(xprof, np.float16)
    T, K = xprof.shape
    perm = np.empty(K, np.int32)
    _check(_lib().woq_outlier_select(_ptr(colsum), _ptr(xprof.view(np.uint16)), T, K, n_out, _ptr(perm)),
           "woq_outlier_select")
    return perm


def woq_outlier_perm(Ws, xprof: np.ndarray, n_out: int = -1) -> np.ndarray:
    """Global permutation of one input space from every linear that reads it
    (float32 [N_l, K] each, in the order given) and its fp16 profile [T, K]."""
    Ws = [np.ascontiguousarray(W, np.float32) for W in Ws]
    xprof = np.ascontiguousarray(xprof, np.float16)
    T, K = xprof.shape
    assert Ws and all(W.ndim == 2 and W.shape[1] == K for W in Ws)
    ptrs = (c_void_p * len(Ws))(*[_ptr(W) for W in Ws])
    ns = (c_int64 * len(Ws))(*[W.shape[0] for W in Ws])
    perm = np.empty(K, np.int32)
    _check(_lib().woq_outlier_perm(ptrs, ns, len(Ws), K, _ptr(xprof.view(np.uint16)), T, n_out, _ptr(perm)),
           "woq_outlier_perm")
    return perm


def woq_outlier_perm_sums(parts, xprof: np.ndarray, n_out: int = -1) -> np.ndarray:
    """Global permutation of one input space from per-linear column sums
    (float64 [K] each, from woq_colabs_accumulate into zeroed buffers), added
    by the library in the order given."""
    parts = [np.ascontiguousarray(p, np.float64) for p in parts]
    xprof = np.ascontiguousarray(xprof, np.float16)
    T, K = xprof.shape
    assert parts and all(p.shape == (K,) for p in parts)
    ptrs = (c_void_p * len(parts))(*[_ptr(p) for p in parts])
    perm = np.empty(K, np.int32)
    _check(_lib().woq_outlier_perm_sums(ptrs, len(parts), K, _ptr(xprof.view(np.uint16)), T, n_out, _ptr(perm)),
           "woq_outlier_perm_sums")
    return perm


def woq_quantize_int4o(W: np.ndarray, perm: np.ndarray, n_out: int = -1):
    W = np.ascontiguousarray(W, np.float32)
    perm = np.ascontiguousarray(perm, np.int32)
    N, K = W.shape
    g = woq_int4o_geometry(K, n_out)
    packed = np.empty((N, g.K_pad // 2), np.uint8)
    scales = np.empty((N, g.G), np.uint16)
    w_out = np.empty((N, g.n_out), np.uint16)
    _check(_lib().woq_quantize_int4o(_ptr(W), N, K, _ptr(perm), g.n_out, _ptr(packed), _ptr(scales), _ptr(w_out)),
           "woq_quantize_int4o")
    return packed, scales.view(np.float16), w_out.view(np.float16)


def woq_unpack_int4(packed: np.ndarray) -> np.ndarray:
    packed = np.ascontiguousarray(packed, np.uint8)
    N, half = packed.shape
    q = np.empty((N, 2 * half), np.int8)
    _check(_lib().woq_unpack_int4(_ptr(packed), N, 2 * half, _ptr(q)), "woq_unpack_int4")
    return q


def woq_layout_int8(q: np.ndarray) -> np.ndarray:
    q = np.ascontiguousarray(q, np.int8)
    N, K = q.shape
    nbytes = _lib().woq_int8_dev_bytes(N, K)
    dev = np.empty(nbytes, np.uint8)
    _check(_lib().woq_layout_int8(_ptr(q), N, K, _ptr(dev)), "woq_layout_int8")
    return dev


def woq_layout_int8_inverse(dev: np.ndarray, N: int, K: int) -> np.ndarray:
    q = np.empty((N, K), np.int8)
    _check(_lib().woq_layout_int8_inverse(_ptr(np.ascontiguousarray(dev, np.uint8)), N, K, _ptr(q)),
           "woq_layout_int8_inverse")
    return q


def woq_int4o_dev_sizes(N: int, g: Int4oGeom):
    a, b, c = c_int64(), c_int64(), c_int64()
    _check(_lib().woq_int4o_dev_sizes(N, ctypes.byref(g), ctypes.byref(a), ctypes.byref(b), ctypes.byref(c)),
           "woq_int4o_dev_sizes")
    return a.value, b.value, c.value


def woq_layout_int4o(packed, scales, w_out, g: Int4oGeom):
    packed = np.ascontiguousarray(packed, np.uint8)
    scales = np.ascontiguousarray(np.asarray(scales).view(np.uint16))
    w_out = np.ascontiguousarray(np.asarray(w_out).view(np.uint16))
    N = packed.shape[0]
    cb, sb, wb = woq_int4o_dev_sizes(N, g)
    dc = np.empty(cb, np.uint8)
    ds = np.empty(sb // 2, np.uint16)
    dw = np.empty(wb // 2, np.uint16)
    _check(_lib().woq_layout_int4o(_ptr(packed), _ptr(scales), _ptr(w_out), N, ctypes.byref(g), _ptr(dc), _ptr(ds),
                                   _ptr(dw) if dw.size else None), "woq_layout_int4o")
    return dc, ds, dw


def woq_layout_int4o_inverse(dc, ds, dw, N: int, g: Int4oGeom):
    packed = np.empty((N, g.K_pad // 2), np.uint8)
    scales = np.empty((N, g.G), np.uint16)
    w_out = np.empty((N, g.n_out), np.uint16)
    _check(_lib().woq_layout_int4o_inverse(_ptr(dc), _ptr(ds), _ptr(dw) if dw.size else None, N, ctypes.byref(g),
                                           _ptr(packed), _ptr(scales), _ptr(w_out)), "woq_layout_int4o_inverse")
    return packed, scales.view(np.float16), w_out.view(np.float16)


# --------------------------------------------------------------- device ops

def need_rows(b: int, *tensors):
    """The library takes plain pointers and cannot see buffer sizes: refuse a
    batch larger than any of the row-major buffers it would read or write."""
    for t in tensors:
        if t is not None and b > t.shape[0]:
            raise ValueError(f"batch {b} exceeds a buffer of {t.shape[0]} rows")


def woq_permute_x(x, perm_dev, g: Int4oGeom, xp, stream=None, ldx: int | None = None):
    b = x.shape[0]
    need_rows(b, xp)
    _check(_lib().woq_permute_x(_ptr(x), ldx or x.shape[1], _ptr(perm_dev), b, ctypes.byref(g), _ptr(xp),
                                _stream(stream)), "woq_permute_x")
    return xp


def woq_qgemv_int8(w: Int8W, x, y, stream=None, b: int | None = None):
    b = x.shape[0] if b is None else b
    need_rows(b, x, y)
    _check(_lib().woq_qgemv_int8(ctypes.byref(w), _ptr(x), x.shape[1], b, _ptr(y), y.shape[1], _stream(stream)),
           "woq_qgemv_int8")
    return y


def woq_quantize_int8_dev(W, dev, scale, status, stream=None):
    """INT8 encoding of the device tensor W (fp32 [N, K]) into the device
    layout ``dev`` (uint8 tensor of woq_int8_dev_bytes) and ``scale`` (fp32
    device tensor [1]); ``status`` (int32 device tensor [1]) receives 0 or
    WOQ_ERANGE."""
    N, K = W.shape
    _check(_lib().woq_quantize_int8_dev(_ptr(W), N, K, _ptr(dev), _ptr(scale), _ptr(status), _stream(stream)),
           "woq_quantize_int8_dev")


def woq_quantize_int4o_dev(W, perm_dev, g: Int4oGeom, codes, scales, w_out, status, stream=None):
    """Outlier-aware INT4 encoding of the device tensor W (fp32 [N, K]) into the
    device layout arrays (torch tensors sized by woq_int4o_dev_sizes)."""
    N = W.shape[0]
    def opt(t):
        return _ptr(t) if t is not None and t.numel() else None
    _check(_lib().woq_quantize_int4o_dev(_ptr(W), N, _ptr(perm_dev), ctypes.byref(g), opt(codes), opt(scales),
                                         opt(w_out), _ptr(status),
                                         _stream(stream)), "woq_quantize_int4o_dev")


def woq_embed_int8(w: Int8W, ids, y, stream=None, b: int | None = None):
    """Look up rows ``ids`` (int32 device tensor [b]) of an INT8 table into y (fp16 [b, ldy])."""
    b = ids.shape[0] if b is None else b
    need_rows(b, ids, y)
    _check(_lib().woq_embed_int8(ctypes.byref(w), _ptr(ids), b, _ptr(y), y.shape[1], _stream(stream)),
           "woq_embed_int8")
    return y


def woq_qgemv_int4o(w: Int4oW, xp, y, stream=None, b: int | None = None):
    b = xp.shape[0] if b is None else b
    need_rows(b, xp, y)
    _check(_lib().woq_qgemv_int4o(ctypes.byref(w), _ptr(xp), b, _ptr(y), y.shape[1], _stream(stream)),
           "woq_qgemv_int4o")
    return y


def woq_perm_positions(perm: np.ndarray, g: Int4oGeom) -> np.ndarray:
    perm = np.ascontiguousarray(perm, np.int32)
    pos = np.empty(-(-g.K // 8) * 8, np.uint16)
    _check(_lib().woq_perm_positions(_ptr(perm), ctypes.byref(g), _ptr(pos)), "woq_perm_positions")
    return pos


def woq_qgemv_int4o_x_supported(g: Int4oGeom, b: int) -> bool:
    return bool(_lib().woq_qgemv_int4o_x_supported(ctypes.byref(g), b))


def woq_qgemv_int4o_x(w: Int4oW, x, pos_dev, y, stream=None, b: int | None = None, ldx: int | None = None):
    b = x.shape[0] if b is None else b
    need_rows(b, x, y)
    _check(_lib().woq_qgemv_int4o_x(ctypes.byref(w), _ptr(x), ldx or x.shape[1], _ptr(pos_dev), b, _ptr(y),
                                    y.shape[1], _stream(stream)), "woq_qgemv_int4o_x")
    return y


def woq_qgemm_int4o_x_supported(g: Int4oGeom, N: int, b: int) -> bool:
    return bool(_lib().woq_qgemm_int4o_x_supported(ctypes.byref(g), N, b))


def woq_qgemm_int4o_x(w: Int4oW, x, pos_dev, y, stream=None, b: int | None = None, ldx: int | None = None):
    """The matrix-core product with the permutation folded in: x in its
    natural channel order, pos_dev the device copy of woq_perm_positions."""
    b = x.shape[0] if b is None else b
    need_rows(b, x, y)
    _check(_lib().woq_qgemm_int4o_x(ctypes.byref(w), _ptr(x), ldx or x.shape[1], _ptr(pos_dev), b, _ptr(y),
                                    y.shape[1], _stream(stream)), "woq_qgemm_int4o_x")
    return y


def woq_stream_read(buf, stream=None):
    """Read every byte of a contiguous device tensor (size a multiple of 16)."""
    _check(_lib().woq_stream_read(_ptr(buf), buf.numel() * buf.element_size(), _stream(stream)), "woq_stream_read")


def woq_dispatch_floor(blocks: int, threads: int, iters: int, stream=None):
    """(span_us, interval_us) of `iters` empty launches of blocks x threads:
    the mean time between each launch's dispatch-boundary events, and the
    mean time per launch back to back."""
    span, interval = ctypes.c_float(), ctypes.c_float()
    _check(_lib().woq_dispatch_floor(blocks, threads, iters, _stream(stream), ctypes.byref(span),
                                     ctypes.byref(interval)), "woq_dispatch_floor")
    return float(span.value), float(interval.value)


def woq_qgemm_int4o_splitk(w: Int4oW, xp, y, splits: int, workspace, stream=None, b: int | None = None):
    """woq_qgemm_int4o over `splits` K ranges; workspace: fp32 device tensor of at
    least woq_qgemm_int4o_splitk_workspace(N, b, splits) bytes."""
    b = xp.shape[0] if b is None else b
    need_rows(b, xp, y)
    _check(_lib().woq_qgemm_int4o_splitk(ctypes.byref(w), _ptr(xp), b, _ptr(y), y.shape[1], splits, _ptr(workspace),
                                         workspace.numel() * workspace.element_size(), _stream(stream)),
           "woq_qgemm_int4o_splitk")
    return y


SPLITK_NOALLOC_BYTES = 8 << 20


def woq_qgemm_int4o_splitk_noalloc(w: Int4oW, xp, y, splits: int, stream=None, b: int | None = None):
    """woq_qgemm_int4o_splitk with the library's fixed per-device workspace
    (no allocation; calls on one device must not overlap)."""
    b = xp.shape[0] if b is None else b
    need_rows(b, xp, y)
    _check(_lib().woq_qgemm_int4o_splitk_noalloc(ctypes.byref(w), _ptr(xp), b, _ptr(y), y.shape[1], splits,
                                                 _stream(stream)), "woq_qgemm_int4o_splitk_noalloc")


def woq_qgemm_int4o(w: Int4oW, xp, y, stream=None, b: int | None = None):
    b = xp.shape[0] if b is None else b
    need_rows(b, xp, y)
    _check(_lib().woq_qgemm_int4o(ctypes.byref(w), _ptr(xp), b, _ptr(y), y.shape[1], _stream(stream)),
           "woq_qgemm_int4o")
    return y


# ------------------------------------------------- device-resident weights

class DeviceInt8:
    """Device layout of one or more INT8 linears stacked along N (one launch).

    ``parts`` is a list of (q int8 [N_i, K], scale) from woq_quantize_int8."""

    def __init__(self, parts, device="cuda"):
        import torch
        K = parts[0][0].shape[1]
        assert all(q.shape[1] == K for q, _ in parts) and len(parts) <= MAX_SEGMENTS
        q = np.concatenate([p[0] for p in parts], axis=0) if len(parts) > 1 else parts[0][0]
        self.N, self.K = q.shape
        self.codes = torch.from_numpy(woq_layout_int8(q)).to(device)
        self.desc = Int8W()
        self.desc.codes = self.codes.data_ptr()
        self.desc.N, self.desc.K, self.desc.nseg = self.N, K, len(parts)
        end = 0
        self.segments = []
        for i, (qi, s) in enumerate(parts):
            end += qi.shape[0]
            self.desc.seg_end[i] = end
            self.desc.seg_scale[i] = float(s)
            self.segments.append((end - qi.shape[0], end))

    @property
    def nbytes(self):
        return int(self.codes.numel())


class DeviceInt4o:
    """Device layout of one or more outlier-INT4 linears of one input space
    stacked along N.  ``parts`` is a list of (packed, scales, w_out) from
    woq_quantize_int4o sharing the geometry ``g``."""

    def __init__(self, parts, g: Int4oGeom, device="cuda"):
        import torch
        packed = np.concatenate([p[0] for p in parts]) if len(parts) > 1 else parts[0][0]
        scales = np.concatenate([p[1] for p in parts]) if len(parts) > 1 else parts[0][1]
        w_out = np.concatenate([p[2] for p in parts]) if len(parts) > 1 else parts[0][2]
        self.N = packed.shape[0]
        self.geom = g
        dc, ds, dw = woq_layout_int4o(packed, scales, w_out, g)
        self.codes = torch.from_numpy(dc).to(device)
        self.scales = torch.from_numpy(ds.view(np.int16)).to(device)
        self.w_out = torch.from_numpy(dw.view(np.int16)).to(device) if dw.size else None
        self.desc = Int4oW()
        self.desc.codes = self.codes.data_ptr()
        self.desc.scales = self.scales.data_ptr()
        self.desc.w_out = self.w_out.data_ptr() if self.w_out is not None else None
        self.desc.N = self.N
        self.desc.geom = g
        self.segments = []
        end = 0
        for p in parts:
            self.segments.append((end, end + p[0].shape[0]))
            end += p[0].shape[0]


# ------------------------------------------------------------- stack runner

class Stack:
    """Owns a woq_stack built from a list of StackStep (weights stay owned by
    the caller, who must keep them alive)."""

    def __init__(self, steps, max_b: int):
        self.steps = (StackStep * len(steps))(*steps)
        self.n = len(steps)
        h = c_void_p()
        _check(_lib().woq_stack_create(self.steps, self.n, max_b, ctypes.byref(h)), "woq_stack_create")
        self.handle = h

    @staticmethod
    def _ptrs(tensors):
        return (c_void_p * len(tensors))(*[t.data_ptr() for t in tensors])

    def bind(self, inputs, outputs):
        """Fix the input/output slot tensors (keeps references).  Every slot a
        step names must be present, and each tensor must be a contiguous fp16
        GPU tensor exactly as wide as the steps that use it (ValueError)."""
        check_slots(slot_widths(self.steps), inputs, outputs)
        self._in, self._out = list(inputs), list(outputs)
        self._pin, self._pout = self._ptrs(self._in), self._ptrs(self._out)

    def run(self, b: int, stream=None):
        need_rows(b, *self._in, *self._out)
        _check(_lib().woq_stack_run(self.handle, self._pin, self._pout, b, _stream(stream)), "woq_stack_run")

    def launches(self, b: int) -> int:
        n = c_int32()
        _check(_lib().woq_stack_launches(self.handle, b, ctypes.byref(n)), "woq_stack_launches")
        return n.value

    def time(self, b: int, iters: int, stream=None):
        need_rows(b, *self._in, *self._out)
        step_ms = (c_float * max(1, self.n))()
        pass_ms = c_float()
        _check(_lib().woq_stack_time(self.handle, self._pin, self._pout, b, _stream(stream), iters, step_ms,
                                     ctypes.byref(pass_ms)), "woq_stack_time")
        return [step_ms[i] for i in range(self.n)], pass_ms.value

    def close(self):
        if getattr(self, "handle", None):
            _check(_lib().woq_stack_destroy(self.handle), "woq_stack_destroy")
            self.handle = None

    def __del__(self):
        # at interpreter shutdown the HIP runtime (or a profiler attached to
        # it) may already be torn down: leave the memory to process exit
        if sys.is_finalizing():
            return
        try:
            self.close()
        except Exception:
            pass


def slot_widths(steps):
    """(in_slot, K, out_slot, N) of every step: StackStep, or PagerStep (an
    all-streamed INT8 pager: step i uses slot i both ways)."""
    out = []
    for i, st in enumerate(steps):
        if isinstance(st, PagerStep):
            out.append((i, int(st.w.K), i, int(st.w.N)))
        elif st.fmt == FMT_INT4O:
            out.append((int(st.in_slot), int(st.w4.geom.K), int(st.out_slot), int(st.w4.N)))
        else:
            out.append((int(st.in_slot), int(st.w8.K), int(st.out_slot), int(st.w8.N)))
    return out


def check_slots(widths, inputs, outputs, device_type: str = "cuda"):
    """Raise ValueError unless every slot a step names is bound to a
    contiguous 2-D fp16 tensor on the GPU (``device_type``) whose rows are
    exactly as wide as that step's input (K) or output (N): the C runner sees
    pointers only, so a missing slot, a narrow or strided tensor would be read
    or written out of bounds on the device."""
    import torch

    def ok(t, width, what, slot):
        if not isinstance(t, torch.Tensor):
            raise ValueError(f"{what} slot {slot}: not a torch tensor")
        if t.device.type != device_type:
            raise ValueError(f"{what} slot {slot}: not on the GPU")
        if t.dtype != torch.float16:
            raise ValueError(f"{what} slot {slot}: dtype {t.dtype}, expected float16")
        if t.dim() != 2 or not t.is_contiguous():
            raise ValueError(f"{what} slot {slot}: must be a contiguous [rows, width] tensor")
        if t.shape[1] != width:
            raise ValueError(f"{what} slot {slot}: width {t.shape[1]}, the step needs {width}")

    for i, (si, K, so, N) in enumerate(widths):
        if not 0 <= si < len(inputs):
            raise ValueError(f"step {i} reads input slot {si}; {len(inputs)} inputs bound")
        if not 0 <= so < len(outputs):
            raise ValueError(f"step {i} writes output slot {so}; {len(outputs)} outputs bound")
        ok(inputs[si], K, "input", si)
        ok(outputs[so], N, "output", so)


def step_int4o(dev: "DeviceInt4o", perm_dev, in_slot: int, out_slot: int) -> StackStep:
    st = StackStep()
    st.fmt, st.in_slot, st.out_slot = FMT_INT4O, in_slot, out_slot
    st.w4 = dev.desc
    st.perm = perm_dev.data_ptr()
    return st


def step_int8(dev: "DeviceInt8", in_slot: int, out_slot: int) -> StackStep:
    st = StackStep()
    st.fmt, st.in_slot, st.out_slot = FMT_INT8, in_slot, out_slot
    st.w8 = dev.desc
    return st


# ------------------------------------------------------------ streamed pager

def woq_pool_save(path: str, meta: bytes, blocks):
    """Write a pool file: ``meta`` bytes and ``blocks`` (NumPy uint8 arrays or
    CPU tensors, contiguous)."""
    n = len(blocks)
    ptrs = (c_void_p * max(1, n))(*[_ptr(b) for b in blocks])
    sizes = (c_int64 * max(1, n))(*[int(b.nbytes if isinstance(b, np.ndarray) else b.numel() * b.element_size())
                                   for b in blocks])
    mbuf = ctypes.create_string_buffer(meta, len(meta)) if meta else None
    _check(_lib().woq_pool_save(os.fsencode(path), mbuf, len(meta), ptrs, sizes, n), "woq_pool_save")


def woq_pool_info(path: str):
    """(meta bytes, [block sizes]) of a pool file."""
    nb, mb = c_int32(), c_int64()
    _check(_lib().woq_pool_info(os.fsencode(path), ctypes.byref(nb), ctypes.byref(mb), None, 0, None, 0),
           "woq_pool_info")
    sizes = (c_int64 * max(1, nb.value))()
    meta = ctypes.create_string_buffer(max(1, mb.value))
    _check(_lib().woq_pool_info(os.fsencode(path), ctypes.byref(nb), ctypes.byref(mb), sizes, nb.value, meta,
                                mb.value), "woq_pool_info")
    return meta.raw[:mb.value], [sizes[i] for i in range(nb.value)]


def woq_pool_read_block(path: str, i: int, dst):
    """Read block i into dst (NumPy uint8 array or contiguous CPU tensor) and verify it."""
    n = dst.nbytes if isinstance(dst, np.ndarray) else dst.numel() * dst.element_size()
    _check(_lib().woq_pool_read_block(os.fsencode(path), i, _ptr(dst), n), "woq_pool_read_block")
    return dst


def woq_plan_tiers(layer_bytes, budget_bytes: int):
    """(resident flags int32 [L], device bytes) of the tier plan under a budget."""
    lb = np.ascontiguousarray(layer_bytes, np.int64)
    res = np.zeros(lb.size, np.int32)
    dev = c_int64()
    _check(_lib().woq_plan_tiers(_ptr(lb), lb.size, int(budget_bytes), _ptr(res), ctypes.byref(dev)),
           "woq_plan_tiers")
    return res, dev.value


class Pager:
    """Owns a woq_pager over a caller-owned pinned pool (kept referenced).

    ``steps`` are PagerStep (INT8 layers, all streamed: woq_pager_create) or
    StackStep (tiered: woq_tiered_create, layer_bytes[l] == 0 marks a resident
    layer, streamed steps carry byte offsets in their weight pointers)."""

    def __init__(self, pool, layer_off, layer_bytes, steps, steps_per_layer: int, max_b: int):
        self.pool = pool
        self.off = (c_int64 * len(layer_off))(*layer_off)
        self.bytes = (c_int64 * len(layer_bytes))(*layer_bytes)
        tiered = isinstance(steps[0], StackStep)
        self.steps = ((StackStep if tiered else PagerStep) * len(steps))(*steps)
        self.n = len(steps)
        h = c_void_p()
        pool_ptr = _ptr(pool) if pool is not None else None
        fn = "woq_tiered_create" if tiered else "woq_pager_create"
        _check(getattr(_lib(), fn)(pool_ptr, self.off, self.bytes, len(layer_off), self.steps, steps_per_layer,
                                   max_b, ctypes.byref(h)), fn)
        self.handle = h

    def bind(self, inputs, outputs):
        """As Stack.bind; an all-streamed INT8 pager's step i reads input slot
        i and writes output slot i."""
        check_slots(slot_widths(self.steps), inputs, outputs)
        self._in, self._out = list(inputs), list(outputs)
        self._pin = (c_void_p * len(self._in))(*[t.data_ptr() for t in self._in])
        self._pout = (c_void_p * len(self._out))(*[t.data_ptr() for t in self._out])

    def run(self, b: int, compute_stream, copy_stream):
        need_rows(b, *self._in, *self._out)
        _check(_lib().woq_pager_run(self.handle, self._pin, self._pout, b, _stream(compute_stream),
                                    _stream(copy_stream)), "woq_pager_run")

    def streamed_layers(self) -> int:
        n = c_int32()
        _check(_lib().woq_pager_streamed_layers(self.handle, ctypes.byref(n)), "woq_pager_streamed_layers")
        return n.value

    def time(self, b: int, compute_stream, copy_stream):
        """One pass with events around every block copy: (wait, start, end)
        times of each streamed layer's copy in ms from the pass's start, and
        the pass's duration."""
        need_rows(b, *self._in, *self._out)
        n = max(1, self.streamed_layers())
        w, c, e, p = (c_float * n)(), (c_float * n)(), (c_float * n)(), c_float()
        _check(_lib().woq_pager_time(self.handle, self._pin, self._pout, b, _stream(compute_stream),
                                     _stream(copy_stream), w, c, e, ctypes.byref(p)), "woq_pager_time")
        k = self.streamed_layers()
        return [w[i] for i in range(k)], [c[i] for i in range(k)], [e[i] for i in range(k)], p.value

    def close(self):
        if getattr(self, "handle", None):
            _check(_lib().woq_pager_destroy(self.handle), "woq_pager_destroy")
            self.handle = None

    def __del__(self):
        if sys.is_finalizing():
            return
        try:
            self.close()
        except Exception:
            pass
