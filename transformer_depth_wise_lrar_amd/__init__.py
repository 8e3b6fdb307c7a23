"""Python binding of liblrattnres, the LR-AttnRes depth-mix read for MI355X (gfx950).

The functions here have the names of the C entry points in include/lrattnres.h and only
marshal arguments: they take torch tensors on the GPU, pass raw device pointers, strides
and the current HIP stream to the library, and allocate outputs with torch when the
caller does not pass them. Every step of the read runs in the library's HIP kernels.

There is no fallback: if liblrattnres.so is missing or cannot be loaded, every call raises
LibraryNotBuilt. Build it with ``python -m transformer_depth_wise_lrar_amd.build``.
"""
from __future__ import annotations

import ctypes
import os
import threading
from typing import Sequence

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "liblrattnres.so")

LRAR_OK, LRAR_ERR_INVALID, LRAR_ERR_UNSUPPORTED, LRAR_ERR_DEVICE = 0, 1, 2, 3
LRAR_F32, LRAR_BF16 = 0, 1
VARIANTS = {"auto": 0, "two_pass": 1, "online": 2}
MAX_SOURCES = 64
MAX_QUERIES = 64


class LibraryNotBuilt(RuntimeError):
    """liblrattnres.so is not built or cannot be loaded."""


class LrarError(RuntimeError):
    """A non-OK status from the library."""

    def __init__(self, status: int, message: str):
        super().__init__(message)
        self.status = status


_lib = None
_lock = threading.Lock()

_i64, _i32, _f64 = ctypes.c_int64, ctypes.c_int32, ctypes.c_double
_vp = ctypes.c_void_p
_vpp = ctypes.POINTER(ctypes.c_void_p)
_i64p = ctypes.POINTER(ctypes.c_int64)


def lib():
    """The loaded library (raises LibraryNotBuilt if it is absent)."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise LibraryNotBuilt(
                    f"{LIB_PATH} is missing; build it with "
                    "`python -m transformer_depth_wise_lrar_amd.build`")
            try:
                L = ctypes.CDLL(LIB_PATH)
            except OSError as e:
                raise LibraryNotBuilt(f"cannot load {LIB_PATH}: {e}") from e
            L.lrar_forward.argtypes = [_i64, _i32, _i32, _f64, _i32, _i32, _vpp, _i64p, _vp,
                                       _vp, _i64, _vp, _i64, _i32, _vp]
            L.lrar_forward_save.argtypes = [_i64, _i32, _i32, _f64, _i32, _i32, _vpp, _i64p, _vp,
                                            _vp, _i64, _vp, _i64, _i32, _vp]
            L.lrar_backward_saved.argtypes = [_i64, _i32, _i32, _i32, _i32, _vpp, _i64p, _vp, _vp,
                                              _i64, _i32, _vp, _i64, _vpp, _i64p, _i32, _vp, _vp,
                                              ctypes.c_size_t, _vp]
            L.lrar_forward_fullrms.argtypes = [_i64, _i32, _i32, _f64, _i32, _i32, _vpp, _i64p,
                                               _vp, _vp, _i64, _vp, _i64, _vp]
            L.lrar_forward_keys.argtypes = [_i64, _i32, _i32, _f64, _i32, _i32, _vpp, _i64p,
                                            _vpp, _i64p, _vp, _vp, _i64, _vp, _i64, _vp]
            L.lrar_forward_stats.argtypes = [_i64, _i32, _i32, _f64, _i32, _i32, _vpp, _i64p,
                                             _i32, _vp, _i64, _vp, _vp, _i64, _vp, _i32, _i64,
                                             _i64, _vp]
            L.lrar_merge.argtypes = [_i64, _i32, _i32, _f64, _i32, _vp, _vp, _vp, _i32, _i64,
                                     _i32, _vpp, _i64p, _vp, _vp, _i64, _vp, _vp, _vp]
            L.lrar_merge_accumulate.argtypes = [_i64, _i32, _i32, _f64, _i32, _vp, _vp, _vp,
                                                _i32, _i64, _vp, _i64, _vp, _i64, _vp, _i64,
                                                _vp, _vp, _i64, _vp, _vp, _vp]
            L.lrar_backward.argtypes = [_i64, _i32, _i32, _f64, _i32, _i32, _vpp, _i64p, _vp,
                                        _vp, _i64, _vpp, _i64p, _i32, _vp, _vp, ctypes.c_size_t,
                                        _vp]
            L.lrar_backward_grad.argtypes = [_i64, _i32, _i32, _f64, _i32, _i32, _vpp, _i64p,
                                             _vp, _i32, _vp, _i64, _vpp, _i64p, _i32, _vp, _vp,
                                             ctypes.c_size_t, _vp]
            L.lrar_backward_noalloc.argtypes = [_i64, _i32, _i32, _f64, _i32, _i32, _vpp, _i64p,
                                                _vp, _i32, _vp, _i64, _vpp, _i64p, _i32, _vp,
                                                _vp]
            L.lrar_backward_workspace_size.argtypes = [_i64, _i32, _i32, _i32]
            L.lrar_backward_workspace_size.restype = ctypes.c_size_t
            L.lrar_copy.argtypes = [_vp, _vp, ctypes.c_size_t, _vp]
            L.lrar_read_stream.argtypes = [_vp, ctypes.c_size_t, _vp, _vp]
            L.lrar_mix_stream.argtypes = [_i64, _i32, _i32, _vpp, _i64p, _i32, _vpp, _i64p,
                                          _i32, _i32, _i32, _i32, _i32, _i32, _i32, _vp]
            L.lrar_read_stream_sink_bytes.argtypes = []
            L.lrar_read_stream_sink_bytes.restype = ctypes.c_size_t
            for fn in ("lrar_forward", "lrar_forward_save", "lrar_backward_saved",
                       "lrar_forward_fullrms", "lrar_forward_keys",
                       "lrar_forward_stats", "lrar_merge", "lrar_merge_accumulate",
                       "lrar_backward", "lrar_backward_grad", "lrar_backward_noalloc",
                       "lrar_copy", "lrar_read_stream", "lrar_mix_stream"):
                getattr(L, fn).restype = ctypes.c_int
            L.lrar_status_string.argtypes = [ctypes.c_int]
            L.lrar_status_string.restype = ctypes.c_char_p
            L.lrar_last_error.restype = ctypes.c_char_p
            L.lrar_version.restype = ctypes.c_char_p
            _lib = L
    return _lib


def exported_symbols() -> list[str]:
    """The C entry points this binding expects the library to export."""
    return ["lrar_forward", "lrar_forward_save", "lrar_backward_saved", "lrar_forward_fullrms",
            "lrar_forward_keys", "lrar_forward_stats",
            "lrar_merge", "lrar_merge_accumulate", "lrar_backward", "lrar_backward_grad",
            "lrar_backward_noalloc", "lrar_backward_workspace_size", "lrar_copy", "lrar_read_stream",
            "lrar_read_stream_sink_bytes", "lrar_mix_stream", "lrar_status_string",
            "lrar_last_error", "lrar_version"]


class Prepared:
    """A library call with its arguments already marshalled: calling it runs only the C entry
    point (so a timed region holds the launch and nothing of the Python marshalling). It keeps
    the tensors it was built from alive; their contents may change between calls."""

    def __init__(self, fn, args, result, keep):
        self._fn, self._args, self.result, self._keep = fn, args, result, keep

    def __call__(self):
        _check(self._fn(*self._args))
        return self.result


def _run(fn, args, result, keep, prepare):
    if prepare:
        return Prepared(fn, args, result, keep)
    _check(fn(*args))
    return result


def _check(status: int):
    if status != LRAR_OK:
        L = lib()
        raise LrarError(status, f"{L.lrar_status_string(status).decode()}: "
                                f"{L.lrar_last_error().decode()}")


def _torch():
    import torch

    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return LRAR_BF16
    if t.dtype == torch.float32:
        return LRAR_F32
    raise TypeError(f"unsupported dtype {t.dtype}; use bfloat16 or float32")


def _rows(t, name):
    if t.dim() != 2 or t.stride(1) != 1:
        raise ValueError(f"{name} must be a 2-D tensor with unit column stride")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    return t.data_ptr(), t.stride(0)


def _need(t, shape, dtype, name):
    """t is a GPU tensor of `dtype` whose leading dims are at least `shape` (None = any).
    Every buffer the library writes or reads is checked here, so a wrongly sized tensor
    fails on the host instead of in a kernel."""
    if not getattr(t, "is_cuda", False):
        raise ValueError(f"{name} must be a GPU tensor")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.dim() != len(shape):
        raise ValueError(f"{name} must have {len(shape)} dims, got shape {tuple(t.shape)}")
    for k, (have, want) in enumerate(zip(t.shape, shape)):
        if want is not None and have < want:
            raise ValueError(f"{name} has shape {tuple(t.shape)}; dim {k} must be >= {want}")
    if t.numel() and t.stride(-1) != 1:
        raise ValueError(f"{name} needs a unit inner stride")
    return t


def _query(q, r, name="q"):
    torch = _torch()
    _need(q, (r,), torch.float32, name)
    return q


def _stream(stream):
    if stream is None:
        return ctypes.c_void_p(_torch().cuda.current_stream().cuda_stream)
    if isinstance(stream, int):
        return ctypes.c_void_p(stream)
    return ctypes.c_void_p(stream.cuda_stream)


def _src_table(srcs: Sequence, io: int | None):
    n = len(srcs)
    if n > MAX_SOURCES:
        raise ValueError(f"at most {MAX_SOURCES} sources")
    ptrs = (ctypes.c_void_p * max(n, 1))()
    lds = (ctypes.c_int64 * max(n, 1))()
    T = d = None
    for i, s in enumerate(srcs):
        if io is not None and _dtype_code(s) != io:
            raise TypeError("all sources must share one dtype")
        io = _dtype_code(s)
        p, ld = _rows(s, f"src[{i}]")
        ptrs[i], lds[i] = p, ld
        if T is None:
            T, d = s.shape
        elif tuple(s.shape) != (T, d):
            raise ValueError("all sources must share one shape")
    return ptrs, lds, io, T, d


def lrar_forward(srcs: Sequence, q, r: int, eps: float = 1e-6, out=None, alpha=None,
                 variant: str = "auto", stream=None, prepare: bool = False):
    """h = sum_i softmax_i(q . RMSNorm(tail_r(o_i))) o_i for every row.

    srcs: n tensors [T, d] (bf16 or fp32, unit column stride); q: fp32 [r].
    out: optional [T, d] of the sources' dtype. alpha: True to return the weights, or an
    fp32 [T, >=n] tensor to write them into. Returns (out, alpha or None)."""
    torch = _torch()
    ptrs, lds, io, T, d = _src_table(srcs, None)
    _query(q, r)
    if out is None:
        out = torch.empty((T, d), dtype=srcs[0].dtype, device=srcs[0].device)
    _need(out, (T, d), srcs[0].dtype, "out")
    op, old = _rows(out, "out")
    if alpha is True:
        alpha = torch.empty((T, len(srcs)), dtype=torch.float32, device=srcs[0].device)
    if alpha is False:
        alpha = None
    if alpha is not None:
        _need(alpha, (T, len(srcs)), torch.float32, "alpha")
    ap, ald = _rows(alpha, "alpha") if alpha is not None else (None, 0)
    args = (T, d, r, float(eps), io, len(srcs), ptrs, lds, q.data_ptr(), op, old, ap, ald,
            VARIANTS[variant], _stream(stream))
    return _run(lib().lrar_forward, args, (out, alpha), (srcs, q, out, alpha), prepare)


def lrar_forward_save(srcs: Sequence, q, r: int, eps: float = 1e-6, out=None, saved=None,
                      variant: str = "auto", stream=None, prepare: bool = False):
    """lrar_forward that also writes the statistics the backward reuses: saved [T, 2n] float64,
    the scores z_i in columns 0..n-1 and 1 / rho_i in columns n..2n-1. Returns (out, saved)."""
    torch = _torch()
    ptrs, lds, io, T, d = _src_table(srcs, None)
    n = len(srcs)
    _query(q, r)
    if out is None:
        out = torch.empty((T, d), dtype=srcs[0].dtype, device=srcs[0].device)
    _need(out, (T, d), srcs[0].dtype, "out")
    if saved is None:
        saved = torch.empty((T, 2 * n), dtype=torch.float64, device=srcs[0].device)
    _need(saved, (T, 2 * n), torch.float64, "saved")
    op, old = _rows(out, "out")
    sp, sld = _rows(saved, "saved")
    args = (T, d, r, float(eps), io, n, ptrs, lds, q.data_ptr(), op, old, sp, sld,
            VARIANTS[variant], _stream(stream))
    return _run(lib().lrar_forward_save, args, (out, saved), (srcs, q, out, saved), prepare)


def _read_outputs(srcs, T, d, out, alpha):
    torch = _torch()
    if out is None:
        out = torch.empty((T, d), dtype=srcs[0].dtype, device=srcs[0].device)
    _need(out, (T, d), srcs[0].dtype, "out")
    if alpha is True:
        alpha = torch.empty((T, len(srcs)), dtype=torch.float32, device=srcs[0].device)
    if alpha is False:
        alpha = None
    if alpha is not None:
        _need(alpha, (T, len(srcs)), torch.float32, "alpha")
    return out, alpha


def lrar_forward_fullrms(srcs: Sequence, q, r: int, eps: float = 1e-6, out=None, alpha=None,
                         stream=None, prepare: bool = False):
    """The full-width-RMS control read: the key tail_r(o_i) is divided by the RMS of the whole
    row o_i. Arguments and result as for lrar_forward (one pass, no variant)."""
    ptrs, lds, io, T, d = _src_table(srcs, None)
    _query(q, r)
    out, alpha = _read_outputs(srcs, T, d, out, alpha)
    op, old = _rows(out, "out")
    ap, ald = _rows(alpha, "alpha") if alpha is not None else (None, 0)
    args = (T, d, r, float(eps), io, len(srcs), ptrs, lds, q.data_ptr(), op, old, ap, ald,
            _stream(stream))
    return _run(lib().lrar_forward_fullrms, args, (out, alpha), (srcs, q, out, alpha), prepare)


def lrar_forward_keys(srcs: Sequence, keys: Sequence, q, r: int, eps: float = 1e-6, out=None,
                      alpha=None, stream=None, prepare: bool = False):
    """The separate-key read: source i routes by the RMS-normalised first r columns of keys[i]
    ([T, >= r], the sources' dtype) and contributes its full row srcs[i] to h. Arguments and
    result otherwise as for lrar_forward (one pass, no variant)."""
    ptrs, lds, io, T, d = _src_table(srcs, None)
    if len(keys) != len(srcs):
        raise ValueError("one key tensor per source")
    kptrs = (ctypes.c_void_p * max(len(keys), 1))()
    klds = (ctypes.c_int64 * max(len(keys), 1))()
    for i, k in enumerate(keys):
        _need(k, (T, r), srcs[0].dtype, f"keys[{i}]")
        kptrs[i], klds[i] = _rows(k, f"keys[{i}]")
    _query(q, r)
    out, alpha = _read_outputs(srcs, T, d, out, alpha)
    op, old = _rows(out, "out")
    ap, ald = _rows(alpha, "alpha") if alpha is not None else (None, 0)
    args = (T, d, r, float(eps), io, len(srcs), ptrs, lds, kptrs, klds, q.data_ptr(), op, old,
            ap, ald, _stream(stream))
    return _run(lib().lrar_forward_keys, args, (out, alpha), (srcs, keys, q, out, alpha),
                prepare)


def lrar_forward_stats(srcs: Sequence, qs, r: int, eps: float = 1e-6, acc_dtype=None,
                       m=None, l=None, acc=None, stream=None, prepare: bool = False):
    """Phase-1 statistics of queries qs [nq, r] against the sources.

    Returns (m [nq, T], l [nq, T], acc [nq, T, d]); acc is unnormalised, fp32 by default."""
    torch = _torch()
    ptrs, lds, io, T, d = _src_table(srcs, None)
    if qs.dim() == 1:
        qs = qs.view(1, -1)
    _need(qs, (1, r), torch.float32, "qs")
    nq = qs.shape[0]
    dev = srcs[0].device
    acc_dtype = torch.float32 if acc_dtype is None else acc_dtype
    if m is None:
        m = torch.empty((nq, T), dtype=torch.float32, device=dev)
    if l is None:
        l = torch.empty((nq, T), dtype=torch.float32, device=dev)
    if acc is None:
        acc = torch.empty((nq, T, d), dtype=acc_dtype, device=dev)
    _need(m, (nq, T), torch.float32, "m")
    _need(l, (nq, T), torch.float32, "l")
    _need(acc, (nq, T, d), None, "acc")
    if acc.stride(2) != 1 or m.stride(1) != 1 or l.stride(1) != 1 or m.stride(0) != l.stride(0):
        raise ValueError("m, l, acc need unit inner stride and m, l one row stride")
    args = (T, d, r, float(eps), io, len(srcs), ptrs, lds, nq, qs.data_ptr(), qs.stride(0),
            m.data_ptr(), l.data_ptr(), m.stride(0), acc.data_ptr(), _dtype_code(acc),
            acc.stride(1), acc.stride(0), _stream(stream))
    return _run(lib().lrar_forward_stats, args, (m, l, acc), (srcs, qs, m, l, acc), prepare)


def lrar_merge(m, l, acc, srcs: Sequence, q, r: int, eps: float = 1e-6, out=None,
               stats_out: bool = False, io_dtype=None, stream=None, prepare: bool = False):
    """Phase-2 merge of one site's statistics (m [T], l [T], acc [T, d]) with extra sources.

    Returns out, or (out, m', l') with stats_out=True."""
    torch = _torch()
    ptrs, lds, io, T, d = _src_table(srcs, None)
    if io is None:
        if out is None and io_dtype is None:
            raise ValueError("with no extra sources pass out= or io_dtype=")
        io = _dtype_code(out) if out is not None else (
            LRAR_BF16 if io_dtype == torch.bfloat16 else LRAR_F32)
    if T is not None and tuple(acc.shape) != (T, d):
        raise ValueError("acc and the extra sources must share one shape [T, d]")
    T, d = acc.shape
    _need(acc, (T, d), None, "acc")
    _need(m, (T,), torch.float32, "m")
    _need(l, (T,), torch.float32, "l")
    if len(srcs):
        _query(q, r)
    if out is None:
        out = torch.empty((T, d), dtype=torch.bfloat16 if io == LRAR_BF16 else torch.float32,
                          device=acc.device)
    _need(out, (T, d), torch.bfloat16 if io == LRAR_BF16 else torch.float32, "out")
    op, old = _rows(out, "out")
    accp, accld = _rows(acc, "acc")
    m_out = l_out = None
    if stats_out:
        m_out = torch.empty((T,), dtype=torch.float32, device=acc.device)
        l_out = torch.empty((T,), dtype=torch.float32, device=acc.device)
    args = (T, d, r, float(eps), io, m.data_ptr(), l.data_ptr(), accp, _dtype_code(acc), accld,
            len(srcs), ptrs, lds, q.data_ptr() if q is not None else None, op, old,
            m_out.data_ptr() if m_out is not None else None,
            l_out.data_ptr() if l_out is not None else None, _stream(stream))
    result = (out, m_out, l_out) if stats_out else out
    return _run(lib().lrar_merge, args, result, (m, l, acc, srcs, q, out, m_out, l_out), prepare)


def lrar_merge_accumulate(m, l, acc, b, o, q, r: int, eps: float = 1e-6, out=None, b_out=None,
                          stats_out: bool = False, stream=None, prepare: bool = False):
    """Phase 2 with the partial-sum update fused in: b_out = b + o (b None: the block's first
    write), then the merge of (m [T], l [T], acc [T, d]) with the single source b_out.

    b_out may be b (or o) itself to update in place. Returns (out, b_out), or
    (out, b_out, m', l') with stats_out=True."""
    torch = _torch()
    T, d = acc.shape
    _need(acc, (T, d), None, "acc")
    _need(m, (T,), torch.float32, "m")
    _need(l, (T,), torch.float32, "l")
    _need(o, (T, d), None, "o")
    dt = o.dtype
    io = _dtype_code(o)
    if b is not None:
        _need(b, (T, d), dt, "b")
    _query(q, r)
    if b_out is None:
        b_out = torch.empty((T, d), dtype=dt, device=o.device)
    _need(b_out, (T, d), dt, "b_out")
    if out is None:
        out = torch.empty((T, d), dtype=dt, device=o.device)
    _need(out, (T, d), dt, "out")
    op, old = _rows(out, "out")
    accp, accld = _rows(acc, "acc")
    bp, bld = _rows(b, "b") if b is not None else (None, 0)
    obp, obld = _rows(o, "o")
    bop, bold = _rows(b_out, "b_out")
    m_out = l_out = None
    if stats_out:
        m_out = torch.empty((T,), dtype=torch.float32, device=acc.device)
        l_out = torch.empty((T,), dtype=torch.float32, device=acc.device)
    args = (T, d, r, float(eps), io, m.data_ptr(), l.data_ptr(), accp, _dtype_code(acc), accld,
            bp, bld, obp, obld, bop, bold, q.data_ptr(), op, old,
            m_out.data_ptr() if m_out is not None else None,
            l_out.data_ptr() if l_out is not None else None, _stream(stream))
    result = (out, b_out, m_out, l_out) if stats_out else (out, b_out)
    return _run(lib().lrar_merge_accumulate, args, result,
                (m, l, acc, b, o, q, out, b_out, m_out, l_out), prepare)


def lrar_backward_workspace_size(T: int, d: int, r: int, n: int) -> int:
    """Bytes of device workspace lrar_backward needs."""
    return int(lib().lrar_backward_workspace_size(T, d, r, n))


def _backward(fn, grad_code, srcs, q, dout, r, eps, dsrc, accumulate, dq, workspace, stream,
              prepare, noalloc=False, saved=None):
    torch = _torch()
    ptrs, lds, io, T, d = _src_table(srcs, None)
    n = len(srcs)
    dev = srcs[0].device
    gdt = dout.dtype
    if dsrc is None:
        dsrc = [torch.zeros((T, d), dtype=gdt, device=dev) if accumulate
                else torch.empty((T, d), dtype=gdt, device=dev) for _ in range(n)]
    if len(dsrc) != n:
        raise ValueError(f"dsrc needs {n} tensors, got {len(dsrc)}")
    _query(q, r)
    _need(dout, (T, d), gdt, "dout")
    dptrs = (ctypes.c_void_p * max(n, 1))()
    dlds = (ctypes.c_int64 * max(n, 1))()
    for i, g in enumerate(dsrc):
        _need(g, (T, d), gdt, f"dsrc[{i}]")
        dptrs[i], dlds[i] = _rows(g, f"dsrc[{i}]")
    if dq is None:
        dq = torch.empty((r,), dtype=torch.float32, device=dev)
    _need(dq, (r,), torch.float32, "dq")
    gp, gld = _rows(dout, "dout")
    if saved is not None:
        _need(saved, (T, 2 * n), torch.float64, "saved")
        sp, sld = _rows(saved, "saved")
        head = (T, d, r, io, n, ptrs, lds, q.data_ptr(), sp, sld, grad_code)
    else:
        head = (T, d, r, float(eps), io, n, ptrs, lds, q.data_ptr())
        if grad_code is not None:
            head = head + (grad_code,)
    if noalloc:
        args = head + (gp, gld, dptrs, dlds, int(bool(accumulate)), dq.data_ptr(),
                       _stream(stream))
        return _run(fn, args, (dsrc, dq), (srcs, q, dout, dsrc, dq), prepare)
    need = lrar_backward_workspace_size(T, d, r, n)
    if workspace is None:
        workspace = torch.empty((max(need, 8),), dtype=torch.uint8, device=dev)
    args = head + (gp, gld, dptrs, dlds, int(bool(accumulate)), dq.data_ptr(),
                   workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                   _stream(stream))
    return _run(fn, args, (dsrc, dq), (srcs, q, dout, dsrc, dq, workspace, saved), prepare)


def lrar_backward(srcs: Sequence, q, dout, r: int, eps: float = 1e-6, dsrc=None,
                  accumulate: bool = False, dq=None, workspace=None, stream=None,
                  prepare: bool = False):
    """Source and query gradients of one read for upstream gradient dout (fp32 [T, d]).

    Returns (dsrc list of fp32 [T, d], dq fp32 [r])."""
    if dout.dtype != _torch().float32:
        raise TypeError("lrar_backward takes float32 gradients; use lrar_backward_grad")
    return _backward(lib().lrar_backward, None, srcs, q, dout, r, eps, dsrc, accumulate, dq,
                     workspace, stream, prepare)


def lrar_backward_grad(srcs: Sequence, q, dout, r: int, eps: float = 1e-6, dsrc=None,
                       accumulate: bool = False, dq=None, workspace=None, stream=None,
                       prepare: bool = False):
    """lrar_backward with the gradients in dout's dtype (bf16 or fp32): dsrc are [T, d] of
    that dtype (bf16 rounded once, after the optional accumulation); dq stays fp32 [r]."""
    return _backward(lib().lrar_backward_grad, _dtype_code(dout), srcs, q, dout, r, eps, dsrc,
                     accumulate, dq, workspace, stream, prepare)


def lrar_backward_saved(srcs: Sequence, q, saved, dout, r: int, dsrc=None,
                        accumulate: bool = False, dq=None, workspace=None, stream=None,
                        prepare: bool = False):
    """lrar_backward_grad from the statistics lrar_forward_save wrote (saved [T, 2n] float64):
    the keys are not scored again. Gradients in dout's dtype; returns (dsrc, dq)."""
    return _backward(lib().lrar_backward_saved, _dtype_code(dout), srcs, q, dout, r, 0.0, dsrc,
                     accumulate, dq, workspace, stream, prepare, saved=saved)


def lrar_backward_noalloc(srcs: Sequence, q, dout, r: int, eps: float = 1e-6, dsrc=None,
                          accumulate: bool = False, dq=None, stream=None, prepare: bool = False):
    """lrar_backward_grad without a workspace: the library's per-device scratch holds the
    query-gradient partials (the call allocates nothing on the device when dsrc and dq are
    given). Calls that overlap on one GPU race on that scratch."""
    return _backward(lib().lrar_backward_noalloc, _dtype_code(dout), srcs, q, dout, r, eps, dsrc,
                     accumulate, dq, None, stream, prepare, noalloc=True)


def lrar_copy(dst, src, stream=None, prepare: bool = False):
    """Plain streaming copy of src into dst (same byte size, 16-byte multiples)."""
    nbytes = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() != nbytes:
        raise ValueError("dst and src must have the same byte size")
    args = (dst.data_ptr(), src.data_ptr(), nbytes, _stream(stream))
    return _run(lib().lrar_copy, args, dst, (dst, src), prepare)


def lrar_mix_stream(srcs: Sequence, out=None, waves_per_cu: int = 8, depth: int = 1,
                    slots: int = 4, rows_per_wave: int = 4, lockstep: int = 0,
                    waves_per_row: int = 1, stream=None, prepare: bool = False):
    """A plain stream with a kernel's traffic: reads srcs (n bf16 tensors [T, d]) and writes
    their mean to each tensor of out (a tensor [T, d], or a list of them, all float32 or all
    bf16; default one bf16 tensor). The reference kernel for the same-traffic bandwidth
    ceiling; the launch shape (waves per CU, sources loaded together, 16-byte units a lane,
    rows per row group per launch, lockstep 0 / per row / per source group, waves sharing a
    row) is the caller's. Returns out."""
    torch = _torch()
    ptrs, lds, io, T, d = _src_table(srcs, LRAR_BF16)
    if out is None:
        out = torch.empty((T, d), dtype=torch.bfloat16, device=srcs[0].device)
    outs = list(out) if isinstance(out, (list, tuple)) else [out]
    if not outs or len(outs) > MAX_SOURCES:
        raise ValueError(f"1 to {MAX_SOURCES} outputs")
    odt = outs[0].dtype
    if odt not in (torch.float32, torch.bfloat16):
        raise TypeError("outputs must be float32 or bfloat16")
    optrs = (ctypes.c_void_p * len(outs))()
    olds = (ctypes.c_int64 * len(outs))()
    for j, o in enumerate(outs):
        _need(o, (T, d), odt, f"out[{j}]")
        optrs[j], olds[j] = _rows(o, f"out[{j}]")
    args = (T, d, len(srcs), ptrs, lds, len(outs), optrs, olds,
            LRAR_F32 if odt == torch.float32 else LRAR_BF16, int(waves_per_cu),
            int(waves_per_row), int(depth), int(slots), int(rows_per_wave), int(lockstep),
            _stream(stream))
    return _run(lib().lrar_mix_stream, args, out, (srcs, outs), prepare)


def lrar_read_stream(src, sink=None, stream=None, prepare: bool = False):
    """Plain streaming read of src (a 16-byte multiple): the read-bandwidth reference.
    Returns the sink (int32 [lrar_read_stream_sink_bytes() / 4]) the kernel folds it into."""
    torch = _torch()
    nbytes = src.numel() * src.element_size()
    if sink is None:
        sink = torch.empty((int(lib().lrar_read_stream_sink_bytes()) // 4,), dtype=torch.int32,
                           device=src.device)
    if sink.numel() * 4 < int(lib().lrar_read_stream_sink_bytes()):
        raise ValueError("sink too small")
    args = (src.data_ptr(), nbytes, sink.data_ptr(), _stream(stream))
    return _run(lib().lrar_read_stream, args, sink, (src, sink), prepare)


def version() -> str:
    return lib().lrar_version().decode()
