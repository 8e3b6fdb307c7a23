"""The oracle: a plain fp64 CPU statement of the LR-AttnRes depth-mix read.

TEST INFRASTRUCTURE ONLY. Only the test suite, the smoke check and the benchmark's
CPU-baseline leg may import this package. The HIP library never calls it, and the two
share no code: the arithmetic lives in ``lrar_oracle.cpp`` (plain loops, IEEE double)
and this module only marshals numpy arrays into it.

Every function takes sources as a list of 2-D float64 arrays of shape [T, d] (row
strides may differ), the site query ``q`` (float64, length r) and ``eps``. The numbers
these functions return are what the GPU path is compared with.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(HERE, "lrar_oracle.cpp")
LIB_PATH = os.path.join(HERE, "liblrar_oracle.so")

_dp = ctypes.POINTER(ctypes.c_double)
_pp = ctypes.POINTER(ctypes.c_void_p)
_i64p = ctypes.POINTER(ctypes.c_int64)


def compile_oracle(src_path: str, lib_path: str, opt: str = "-O2") -> str:
    """g++ (no fast-math) build of an oracle source file into a shared library."""
    tmp = lib_path + ".tmp%d" % os.getpid()
    subprocess.check_call(["g++", opt, "-std=c++17", "-fPIC", "-shared", "-fno-fast-math",
                           "-Wall", src_path, "-o", tmp])
    os.replace(tmp, lib_path)
    return lib_path


def build(force: bool = False) -> str:
    """Compile lrar_oracle.cpp into liblrar_oracle.so (only when stale, unless forced)."""
    if force or not os.path.exists(LIB_PATH) or (
        os.path.getmtime(LIB_PATH) < os.path.getmtime(SOURCE)
    ):
        compile_oracle(SOURCE, LIB_PATH)
    return LIB_PATH


def _dptr(a):
    return a.ctypes.data_as(_dp) if a is not None else None


def _f64(a):
    a = np.asarray(a)
    if a.dtype != np.float64:
        a = a.astype(np.float64)
    return a


def _src_arrays(srcs):
    """Float64 [T, d] arrays with unit column stride; returns (arrays, ptrs, lds, T, d)."""
    arrs = []
    for s in srcs:
        s = _f64(s)
        if s.ndim != 2:
            raise ValueError("each source must be 2-D [T, d]")
        if s.strides[1] != 8 or s.strides[0] % 8:
            s = np.ascontiguousarray(s)
        arrs.append(s)
    if not arrs:
        return arrs, None, None, 0, 0
    T, d = arrs[0].shape
    for s in arrs:
        if s.shape != (T, d):
            raise ValueError("all sources must share one shape")
    ptrs = (ctypes.c_void_p * len(arrs))(*[s.ctypes.data for s in arrs])
    lds = (ctypes.c_int64 * len(arrs))(*[s.strides[0] // 8 for s in arrs])
    return arrs, ptrs, lds, T, d


def _check(rc, name):
    if rc != 0:
        raise ValueError(f"oracle {name}: invalid arguments")


class Oracle:
    """The oracle's functions bound to one compiled library."""

    def __init__(self, lib_path: str):
        lib = ctypes.CDLL(lib_path)
        i64, i32, dbl = ctypes.c_int64, ctypes.c_int, ctypes.c_double
        lib.orc_scores.argtypes = [i64, i32, i32, dbl, i32, _pp, _i64p, _dp, _dp, _dp]
        lib.orc_forward.argtypes = [i64, i32, i32, dbl, i32, _pp, _i64p, _dp, _dp, i64, _dp]
        lib.orc_attnres_standard.argtypes = [i64, i32, dbl, i32, _pp, _i64p, _dp, _dp, i64,
                                             _dp]
        lib.orc_forward_fullrms.argtypes = lib.orc_forward.argtypes
        lib.orc_forward_keys.argtypes = [i64, i32, i32, dbl, i32, _pp, _i64p, _pp, _i64p, _dp,
                                         _dp, i64, _dp]
        lib.orc_stats.argtypes = [i64, i32, i32, dbl, i32, _pp, _i64p, i32, _dp, _dp, _dp, _dp]
        lib.orc_merge.argtypes = [i64, i32, i32, dbl, _dp, _dp, _dp, i32, _pp, _i64p, _dp, _dp,
                                  i64, _dp, _dp]
        lib.orc_merge_accumulate.argtypes = [i64, i32, i32, dbl, i32, _dp, _dp, _dp, _dp, i64,
                                             _dp, i64, _dp, _dp, _dp, i64, _dp, _dp]
        lib.orc_round_to_format.argtypes = [i64, _dp, i32, _dp]
        lib.orc_backward.argtypes = [i64, i32, i32, dbl, i32, _pp, _i64p, _dp, _dp, i64, _pp,
                                     _dp]
        lib.orc_backward_fullrms.argtypes = lib.orc_backward.argtypes
        for fn in ("orc_scores", "orc_forward", "orc_attnres_standard", "orc_forward_fullrms",
                   "orc_forward_keys", "orc_merge_accumulate", "orc_round_to_format",
                   "orc_stats", "orc_merge", "orc_backward", "orc_backward_fullrms"):
            getattr(lib, fn).restype = ctypes.c_int
        self.lib = lib
        self.path = lib_path

    def scores(self, srcs, q, r, eps):
        """(z, rho), both [T, n]: per-token score and slice RMS of every source."""
        arrs, ptrs, lds, T, d = _src_arrays(srcs)
        q = np.ascontiguousarray(_f64(q))
        n = len(arrs)
        z = np.empty((T, n))
        rho = np.empty((T, n))
        _check(self.lib.orc_scores(T, d, r, eps, n, ptrs, lds, _dptr(q), _dptr(z), _dptr(rho)),
               "scores")
        return z, rho

    def _fwd(self, fn, srcs, q, r, eps, name):
        arrs, ptrs, lds, T, d = _src_arrays(srcs)
        q = np.ascontiguousarray(_f64(q))
        n = len(arrs)
        out = np.empty((T, d))
        alpha = np.empty((T, n))
        _check(fn(T, d, r, eps, n, ptrs, lds, _dptr(q), _dptr(out), d, _dptr(alpha)), name)
        return out, alpha

    def forward(self, srcs, q, r, eps):
        """(h [T, d], alpha [T, n]) of the sliced read."""
        return self._fwd(self.lib.orc_forward, srcs, q, r, eps, "forward")

    def forward_fullrms(self, srcs, q, r, eps):
        """(h, alpha) of the full-width-RMS control read."""
        return self._fwd(self.lib.orc_forward_fullrms, srcs, q, r, eps, "forward_fullrms")

    def forward_keys(self, srcs, keys, q, r, eps):
        """(h, alpha) of the separate-key read: keys is a list of n [T, >= r] arrays whose
        first r columns are the sources' keys."""
        arrs, ptrs, lds, T, d = _src_arrays(srcs)
        karrs = []
        for k in keys:
            k = _f64(k)
            if k.ndim != 2 or k.shape[0] != T or k.shape[1] < r:
                raise ValueError("each key must be [T, >= r]")
            if k.strides[1] != 8 or k.strides[0] % 8:
                k = np.ascontiguousarray(k)
            karrs.append(k)
        if len(karrs) != len(arrs):
            raise ValueError("one key per source")
        n = len(arrs)
        kptrs = (ctypes.c_void_p * n)(*[k.ctypes.data for k in karrs])
        klds = (ctypes.c_int64 * n)(*[k.strides[0] // 8 for k in karrs])
        q = np.ascontiguousarray(_f64(q))
        out = np.empty((T, d))
        alpha = np.empty((T, n))
        _check(self.lib.orc_forward_keys(T, d, r, eps, n, ptrs, lds, kptrs, klds, _dptr(q),
                                         _dptr(out), d, _dptr(alpha)), "forward_keys")
        return out, alpha

    def attnres_standard(self, srcs, q, eps):
        """(h, alpha) of standard AttnRes: full-width key, q of length d."""
        arrs, ptrs, lds, T, d = _src_arrays(srcs)
        q = np.ascontiguousarray(_f64(q))
        n = len(arrs)
        out = np.empty((T, d))
        alpha = np.empty((T, n))
        _check(self.lib.orc_attnres_standard(T, d, eps, n, ptrs, lds, _dptr(q), _dptr(out), d,
                                             _dptr(alpha)), "attnres_standard")
        return out, alpha

    def stats(self, srcs, qs, r, eps):
        """Phase-1 statistics for queries qs [nq, r]: (m [nq, T], l [nq, T], acc [nq, T, d])."""
        arrs, ptrs, lds, T, d = _src_arrays(srcs)
        qs = np.ascontiguousarray(_f64(qs)).reshape(-1, r)
        nq = qs.shape[0]
        n = len(arrs)
        m = np.empty((nq, T))
        l = np.empty((nq, T))
        acc = np.empty((nq, T, d))
        _check(self.lib.orc_stats(T, d, r, eps, n, ptrs, lds, nq, _dptr(qs), _dptr(m),
                                  _dptr(l), _dptr(acc)), "stats")
        return m, l, acc

    def merge(self, m, l, acc, srcs, q, r, eps):
        """Phase-2 merge of (m [T], l [T], acc [T, d]) with extra sources: (h, m', l')."""
        m = np.ascontiguousarray(_f64(m))
        l = np.ascontiguousarray(_f64(l))
        acc = np.ascontiguousarray(_f64(acc))
        T, d = acc.shape
        arrs, ptrs, lds, _, _ = _src_arrays(srcs)
        n = len(arrs)
        q = np.ascontiguousarray(_f64(q)) if q is not None else np.zeros(r)
        out = np.empty((T, d))
        m_out = np.empty(T)
        l_out = np.empty(T)
        _check(self.lib.orc_merge(T, d, r, eps, _dptr(m), _dptr(l), _dptr(acc), n, ptrs, lds,
                                  _dptr(q), _dptr(out), d, _dptr(m_out), _dptr(l_out)),
               "merge")
        return out, m_out, l_out

    def merge_accumulate(self, m, l, acc, b, o, q, r, eps, bits):
        """Phase 2 with the partial-sum update fused in: b' = round(b + o) to a `bits`-bit
        significand (b None: the block's first write), then the merge of (m [T], l [T],
        acc [T, d]) with the single source b'. Returns (h, b', m', l')."""
        m = np.ascontiguousarray(_f64(m))
        l = np.ascontiguousarray(_f64(l))
        acc = np.ascontiguousarray(_f64(acc))
        T, d = acc.shape
        o = np.ascontiguousarray(_f64(o))
        if b is not None:
            b = np.ascontiguousarray(_f64(b))
        q = np.ascontiguousarray(_f64(q))
        b_out = np.empty((T, d))
        out = np.empty((T, d))
        m_out = np.empty(T)
        l_out = np.empty(T)
        _check(self.lib.orc_merge_accumulate(
            T, d, r, eps, bits, _dptr(m), _dptr(l), _dptr(acc), _dptr(b), d, _dptr(o), d,
            _dptr(q), _dptr(b_out), _dptr(out), d, _dptr(m_out), _dptr(l_out)),
            "merge_accumulate")
        return out, b_out, m_out, l_out

    def round_to_format(self, x, bits):
        """x rounded to a `bits`-bit significand, ties to even (24: float32, 8: bfloat16)."""
        x = np.ascontiguousarray(_f64(x))
        y = np.empty_like(x)
        _check(self.lib.orc_round_to_format(x.size, _dptr(x), bits, _dptr(y)), "round")
        return y

    def _bwd(self, fn, srcs, q, dout, r, eps):
        arrs, ptrs, lds, T, d = _src_arrays(srcs)
        q = np.ascontiguousarray(_f64(q))
        dout = _f64(dout)
        if dout.strides[1] != 8 or dout.strides[0] % 8:
            dout = np.ascontiguousarray(dout)
        n = len(arrs)
        dsrc = [np.empty((T, d)) for _ in range(n)]
        dptrs = (ctypes.c_void_p * n)(*[g.ctypes.data for g in dsrc])
        dq = np.empty(r)
        _check(fn(T, d, r, eps, n, ptrs, lds, _dptr(q), _dptr(dout), dout.strides[0] // 8,
                  dptrs, _dptr(dq)), "backward")
        return dsrc, dq

    def backward(self, srcs, q, dout, r, eps):
        """(dsrc list of [T, d], dq [r]) for upstream gradient dout [T, d]."""
        return self._bwd(self.lib.orc_backward, srcs, q, dout, r, eps)

    def backward_fullrms(self, srcs, q, dout, r, eps):
        """Backward of the full-width-RMS control read."""
        return self._bwd(self.lib.orc_backward_fullrms, srcs, q, dout, r, eps)


def block_ends(M: int, N: int) -> list:
    """Last write of each of the N blocks over M sub-layer writes: ceil(M j / N), j = 1..N
    (the author's explainer, "The mechanism in PyTorch-style code", block-end rule)."""
    return [-(-M * j // N) for j in range(1, N + 1)]


def block_sources(M: int, N: int, w: int) -> list:
    """The sources a read sees after write w (0 <= w <= M) under block routing, each as the list
    of writes summed into it (0 = the embedding): the embedding, every completed block as one
    sum, and the writes of the unfinished block if there are any (the explainer, "Full history
    or a few block summaries"; an empty partial sum is not a source). With N = M every write is
    its own source: full routing."""
    if not (0 <= w <= M and 1 <= N <= M):
        raise ValueError("need 0 <= w <= M and 1 <= N <= M")
    out = [[0]]
    start = 1
    for end in block_ends(M, N):
        if end <= w:
            out.append(list(range(start, end + 1)))
            start = end + 1
        else:
            break
    if start <= w:
        out.append(list(range(start, w + 1)))
    return out


_default = None
_lock = threading.Lock()


def default() -> Oracle:
    """The oracle built from lrar_oracle.cpp (compiled on first use if missing)."""
    global _default
    with _lock:
        if _default is None:
            build()
            _default = Oracle(LIB_PATH)
    return _default


def scores(*a, **k):
    return default().scores(*a, **k)


def forward(*a, **k):
    return default().forward(*a, **k)


def forward_fullrms(*a, **k):
    return default().forward_fullrms(*a, **k)


def forward_keys(*a, **k):
    return default().forward_keys(*a, **k)


def merge_accumulate(*a, **k):
    return default().merge_accumulate(*a, **k)


def round_to_format(*a, **k):
    return default().round_to_format(*a, **k)


def attnres_standard(*a, **k):
    return default().attnres_standard(*a, **k)


def stats(*a, **k):
    return default().stats(*a, **k)


def merge(*a, **k):
    return default().merge(*a, **k)


def backward(*a, **k):
    return default().backward(*a, **k)


def backward_fullrms(*a, **k):
    return default().backward_fullrms(*a, **k)
