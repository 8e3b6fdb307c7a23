"""The C-ABI library: it loads, exports every declared entry point, and rejects bad
arguments with a status before touching the device (CPU only; no compute calls)."""
import ctypes
import os
import re

import pytest

import transformer_depth_wise_lrar_amd as lrar

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "lrattnres.h")


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(lrar_[a-z_0-9]+)\s*\(", text)))


@pytest.fixture(scope="module")
def L():
    try:
        return lrar.lib()
    except lrar.LibraryNotBuilt as e:
        pytest.fail(f"library not built: {e}")


def test_every_declared_symbol_is_exported(L):
    names = header_functions()
    assert len(names) >= 9
    for n in names:
        assert hasattr(L, n), n
    assert sorted(lrar.exported_symbols()) == names


def test_version_and_status_strings(L):
    assert L.lrar_version().decode().count(".") == 2
    for s in range(4):
        assert L.lrar_status_string(s)


FAKE = 1 << 20  # a non-null, 16-byte aligned host value; never dereferenced


def _src(n, ld):
    k = max(n, 1)
    return (ctypes.c_void_p * k)(*([FAKE] * k)), (ctypes.c_int64 * k)(*([ld] * k))


def fwd(L, T=4, d=8, r=4, eps=1e-6, io=1, n=2, ld=8, q=FAKE, out=FAKE * 2, out_ld=8,
        alpha=None, alpha_ld=0, variant=0):
    p, l = _src(n, ld)
    return L.lrar_forward(T, d, r, eps, io, n, p, l, q, out, out_ld, alpha, alpha_ld, variant,
                          None)


@pytest.mark.parametrize("kw", [
    dict(T=-1), dict(d=0), dict(r=0), dict(r=9), dict(eps=-1.0), dict(eps=float("nan")),
    dict(eps=float("inf")), dict(io=7), dict(n=0), dict(n=65), dict(ld=7), dict(q=None),
    dict(out=None), dict(out_ld=7), dict(alpha=FAKE * 3, alpha_ld=1), dict(variant=3),
    dict(out=FAKE),  # out aliases a source
])
def test_forward_rejects(L, kw):
    assert fwd(L, **kw) == lrar.LRAR_ERR_INVALID
    assert L.lrar_last_error().decode().startswith("lrar_forward")


def test_forward_empty_is_ok_without_device(L):
    assert fwd(L, T=0) == lrar.LRAR_OK


def fwd_full(L, T=4, d=8, r=4, eps=1e-6, io=1, n=2, ld=8, q=FAKE, out=FAKE * 2, out_ld=8,
             alpha=None, alpha_ld=0):
    p, l = _src(n, ld)
    return L.lrar_forward_fullrms(T, d, r, eps, io, n, p, l, q, out, out_ld, alpha, alpha_ld,
                                  None)


@pytest.mark.parametrize("kw", [
    dict(T=-1), dict(r=0), dict(r=9), dict(eps=-1.0), dict(io=7), dict(n=0), dict(n=65),
    dict(ld=7), dict(q=None), dict(out=None), dict(out_ld=7), dict(alpha=FAKE * 3, alpha_ld=1),
    dict(out=FAKE),
])
def test_forward_fullrms_rejects(L, kw):
    assert fwd_full(L, **kw) == lrar.LRAR_ERR_INVALID
    assert L.lrar_last_error().decode().startswith("lrar_forward_fullrms")


def test_forward_fullrms_limits(L):
    assert fwd_full(L, T=0) == lrar.LRAR_OK
    # rows wider than a register tile take the column-chunked kernel
    assert fwd_full(L, T=0, d=16392, r=16, ld=16392, out_ld=16392) == lrar.LRAR_OK


def fwd_keys(L, T=4, d=8, r=4, io=1, n=2, ld=8, key=FAKE * 4, key_ld=8, keys=True, q=FAKE,
             out=FAKE * 2, out_ld=8):
    p, l = _src(n, ld)
    k = max(n, 1)
    kp = (ctypes.c_void_p * k)(*([key] * k)) if keys else None
    kl = (ctypes.c_int64 * k)(*([key_ld] * k)) if keys else None
    return L.lrar_forward_keys(T, d, r, 1e-6, io, n, p, l, kp, kl, q, out, out_ld, None, 0, None)


@pytest.mark.parametrize("kw", [
    dict(keys=False), dict(key=None), dict(key_ld=3), dict(key=FAKE * 2),  # aliases out
    dict(r=0), dict(r=9), dict(q=None), dict(n=0),
])
def test_forward_keys_rejects(L, kw):
    assert fwd_keys(L, **kw) == lrar.LRAR_ERR_INVALID
    assert L.lrar_last_error().decode().startswith("lrar_forward_keys")


def test_forward_keys_limits(L):
    assert fwd_keys(L, T=0) == lrar.LRAR_OK
    # keys that no spread piece serves (misaligned pieces, r = 1000) and rows wider than a
    # tile take the column-chunked kernel, which reads the keys element by element
    big = dict(T=0, d=1024, r=96, ld=1024, out_ld=1024, key_ld=96)
    assert fwd_keys(L, **big) == lrar.LRAR_OK
    assert fwd_keys(L, key=FAKE * 4 + 2, **big) == lrar.LRAR_OK
    assert fwd_keys(L, key=FAKE * 4 + 2, **dict(big, r=64, key_ld=64)) == lrar.LRAR_OK
    assert fwd_keys(L, **dict(big, r=1000, key_ld=1000)) == lrar.LRAR_OK
    assert fwd_keys(L, **dict(big, d=16392, ld=16392, out_ld=16392)) == lrar.LRAR_OK


def merge_acc(L, T=4, d=8, r=4, io=1, acc_dtype=0, acc_ld=8, b=FAKE * 7, b_ld=8, o=FAKE * 8,
              o_ld=8, b_out=FAKE * 9, b_out_ld=8, q=FAKE * 2, out=FAKE * 6, out_ld=8,
              m_out=None, l_out=None):
    return L.lrar_merge_accumulate(T, d, r, 1e-6, io, FAKE * 3, FAKE * 4, FAKE * 5, acc_dtype,
                                   acc_ld, b, b_ld, o, o_ld, b_out, b_out_ld, q, out, out_ld,
                                   m_out, l_out, None)


@pytest.mark.parametrize("kw", [
    dict(r=0), dict(acc_dtype=5), dict(acc_ld=7), dict(o=None), dict(o_ld=7), dict(b_ld=7),
    dict(b_out=None), dict(b_out_ld=7), dict(q=None), dict(out=None), dict(out_ld=7),
    dict(m_out=FAKE * 10, l_out=FAKE * 10),
    dict(b_out=FAKE * 8 + 16),           # partly overlaps o
    dict(b_out=FAKE * 7, b_out_ld=16),   # starts at b with another row stride
    dict(out=FAKE * 9),                  # out is b_out
    dict(out=FAKE * 8 + 2),              # out overlaps o
])
def test_merge_accumulate_rejects(L, kw):
    assert merge_acc(L, **kw) == lrar.LRAR_ERR_INVALID
    assert L.lrar_last_error().decode().startswith("lrar_merge_accumulate")


def test_merge_accumulate_in_place_and_limits(L):
    assert merge_acc(L, T=0) == lrar.LRAR_OK
    assert merge_acc(L, T=0, b_out=FAKE * 7) == lrar.LRAR_OK   # in place over b
    assert merge_acc(L, T=0, b_out=FAKE * 8) == lrar.LRAR_OK   # in place over o
    assert merge_acc(L, T=0, b=None) == lrar.LRAR_OK           # the block's first write
    wide = dict(T=0, d=16392, acc_ld=16392, b_ld=16392, o_ld=16392, b_out_ld=16392,
                out_ld=16392)
    assert merge_acc(L, **wide) == lrar.LRAR_OK  # an add kernel, then the column-chunked merge


def test_online_too_wide_is_unsupported(L):
    # 2049 units of 8 bf16 are 33 chunks of 64 lanes, one more than a register tile holds
    assert fwd(L, d=16392, r=16, ld=16392, out_ld=16392, variant=2) == \
        lrar.LRAR_ERR_UNSUPPORTED


def stats(L, T=4, d=8, r=4, n=2, nq=3, q_ld=4, ml_ld=4, acc_ld=8, qstride=32, acc_dtype=0,
          m=FAKE * 3, l=FAKE * 4, acc=FAKE * 5):
    p, ld = _src(n, 8)
    return L.lrar_forward_stats(T, d, r, 1e-6, 1, n, p, ld, nq, FAKE * 2, q_ld, m, l, ml_ld, acc,
                                acc_dtype, acc_ld, qstride, None)


@pytest.mark.parametrize("kw", [
    dict(nq=0), dict(nq=65), dict(q_ld=3), dict(ml_ld=3), dict(acc_ld=7), dict(qstride=31),
    dict(acc_dtype=5), dict(m=None), dict(m=FAKE * 4), dict(acc=FAKE),
])
def test_stats_rejects(L, kw):
    assert stats(L, **kw) == lrar.LRAR_ERR_INVALID


def merge(L, T=4, d=8, r=4, n=1, acc_ld=8, out=FAKE * 6, q=FAKE * 2, m_out=None, l_out=None):
    p, ld = _src(n, 8)
    return L.lrar_merge(T, d, r, 1e-6, 1, FAKE * 3, FAKE * 4, FAKE * 5, 0, acc_ld, n, p, ld, q,
                        out, 8, m_out, l_out, None)


@pytest.mark.parametrize("kw", [
    dict(n=-1), dict(acc_ld=7), dict(q=None), dict(out=None), dict(out=FAKE),
    dict(m_out=FAKE * 7, l_out=FAKE * 7),
])
def test_merge_rejects(L, kw):
    assert merge(L, **kw) == lrar.LRAR_ERR_INVALID


def test_merge_without_extra_sources_needs_no_query(L):
    assert merge(L, T=0, n=0, q=None) == lrar.LRAR_OK


def bwd(L, T=4, d=8, r=4, n=2, dsrc=None, accumulate=0, ws=FAKE * 9, ws_bytes=1 << 30,
        dq=FAKE * 8, dout=FAKE * 7):
    p, ld = _src(n, 8)
    dsrc = dsrc if dsrc is not None else [FAKE * (10 + i) for i in range(n)]
    dp = (ctypes.c_void_p * n)(*dsrc)
    dl = (ctypes.c_int64 * n)(*([8] * n))
    return L.lrar_backward(T, d, r, 1e-6, 1, n, p, ld, FAKE * 2, dout, 8, dp, dl, accumulate, dq,
                           ws, ws_bytes, None)


@pytest.mark.parametrize("kw", [
    dict(dsrc=[FAKE * 10, FAKE * 10]), dict(dsrc=[FAKE, FAKE * 11]), dict(accumulate=2),
    dict(ws_bytes=8), dict(ws=None), dict(dq=None), dict(dout=FAKE * 10),
])
def test_backward_rejects(L, kw):
    assert bwd(L, **kw) == lrar.LRAR_ERR_INVALID


def bwd_grad(L, T=4, d=8, r=4, n=2, grad=1, dsrc=None, accumulate=0, dq=FAKE * 8,
             dout=FAKE * 7):
    p, ld = _src(n, 8)
    dsrc = dsrc if dsrc is not None else [FAKE * (10 + i) for i in range(n)]
    dp = (ctypes.c_void_p * n)(*dsrc)
    dl = (ctypes.c_int64 * n)(*([8] * n))
    return L.lrar_backward_grad(T, d, r, 1e-6, 1, n, p, ld, FAKE * 2, grad, dout, 8, dp, dl,
                                accumulate, dq, FAKE * 9, 1 << 30, None)


@pytest.mark.parametrize("kw", [
    dict(grad=7), dict(dsrc=[FAKE * 10, FAKE * 10]), dict(dsrc=[FAKE, FAKE * 11]),
    dict(accumulate=2), dict(dq=None), dict(dout=FAKE * 10), dict(dout=None),
])
def test_backward_grad_rejects(L, kw):
    assert bwd_grad(L, **kw) == lrar.LRAR_ERR_INVALID
    assert L.lrar_last_error().decode().startswith("lrar_backward_grad")


def test_backward_grad_empty_is_ok(L):
    for grad in (0, 1):
        assert bwd_grad(L, T=0, grad=grad) == lrar.LRAR_OK


def test_backward_workspace_size(L):
    assert L.lrar_backward_workspace_size(0, 8, 4, 2) == 0
    a = L.lrar_backward_workspace_size(16384, 4096, 1024, 10)
    assert a > 0 and a % 8 == 0
    assert L.lrar_backward_workspace_size(16384, 4096, 2048, 10) > a


@pytest.mark.parametrize("d,r,ld", [
    (20000, 20000, 20000),  # vector rows past a tile: the key spans 40 chunks (at most 8)
    (20000, 4104, 20000),   # the same, 9 chunks
    (8192, 8192, 8193),     # element path (odd stride): 128 chunks (at most 64)
    (4097, 4097, 4097),     # element path, unaligned width: 65 chunks
])
def test_backward_key_too_wide_is_unsupported(L, d, r, ld):
    """Rows that no row tile holds keep query-gradient partials for the key's chunks of 64
    units in registers; a key spanning more of them is refused, at T > 0, before any device
    work."""
    p, lds_ = _src(1, ld)
    dp = (ctypes.c_void_p * 1)(FAKE * 100)
    dl = (ctypes.c_int64 * 1)(ld)
    assert L.lrar_backward(4, d, r, 1e-6, 1, 1, p, lds_, FAKE * 2, FAKE * 300, ld, dp, dl, 0,
                           FAKE * 4, FAKE * 5, 1 << 30, None) == lrar.LRAR_ERR_UNSUPPORTED
    assert "chunks" in L.lrar_last_error().decode()


# ---- partial overlaps: every output is checked by byte range against every other buffer ----
# Sources sit at FAKE (rows of 8 bf16 = 16 bytes, 4 rows); an offset of 16 bytes starts one row in.

@pytest.mark.parametrize("kw,what", [
    (dict(out=FAKE + 16), "out overlaps src"),                     # out one row into a source
    (dict(out=FAKE + 48 + 8), "out overlaps src"),                 # into the last row's tail
    (dict(alpha=FAKE + 8, alpha_ld=2), "alpha overlaps src"),
    (dict(alpha=FAKE * 2 + 32, alpha_ld=2), "alpha overlaps out"),
    (dict(q=FAKE * 2 + 4), "out overlaps q"),
])
def test_forward_rejects_partial_overlaps(L, kw, what):
    assert fwd(L, **kw) == lrar.LRAR_ERR_INVALID
    assert what in L.lrar_last_error().decode()


def test_forward_keys_rejects_partial_overlap(L):
    assert fwd_keys(L, key=FAKE * 2 + 16) == lrar.LRAR_ERR_INVALID
    assert "out overlaps key" in L.lrar_last_error().decode()


@pytest.mark.parametrize("kw,what", [
    (dict(acc=FAKE + 32), "acc overlaps src"),
    (dict(m=FAKE * 4 - 8), "l overlaps m"),
    (dict(acc=FAKE * 2 + 16), "acc overlaps q"),
    (dict(m=FAKE * 5 + 100), "acc overlaps m"),
])
def test_stats_rejects_partial_overlaps(L, kw, what):
    assert stats(L, **kw) == lrar.LRAR_ERR_INVALID
    assert what in L.lrar_last_error().decode()


@pytest.mark.parametrize("kw,what", [
    (dict(out=FAKE + 16), "out overlaps src"),
    (dict(out=FAKE * 5 + 64), "out overlaps acc"),
    (dict(m_out=FAKE * 3 + 4), "m_out overlaps m"),
    (dict(m_out=FAKE * 7, l_out=FAKE * 7 + 8), "l_out overlaps m_out"),
])
def test_merge_rejects_partial_overlaps(L, kw, what):
    assert merge(L, **kw) == lrar.LRAR_ERR_INVALID
    assert what in L.lrar_last_error().decode()


@pytest.mark.parametrize("kw,what", [
    (dict(dsrc=[FAKE * 10, FAKE * 10 + 64]), "dsrc[1] overlaps dsrc[0]"),
    (dict(dsrc=[FAKE * 7 + 32, FAKE * 11]), "dsrc[0] overlaps dout"),
    (dict(dsrc=[FAKE + 16, FAKE * 11]), "dsrc[0] overlaps src"),
    (dict(dq=FAKE * 10 + 4), "dq overlaps dsrc[0]"),
    (dict(ws=FAKE * 7 + 16), "workspace overlaps dout"),
])
def test_backward_rejects_partial_overlaps(L, kw, what):
    assert bwd(L, **kw) == lrar.LRAR_ERR_INVALID
    assert what in L.lrar_last_error().decode()


def test_copy_rejects(L):
    assert L.lrar_copy(FAKE, FAKE + 8, 64, None) == lrar.LRAR_ERR_INVALID
    assert L.lrar_copy(FAKE, FAKE + 16, 64, None) == lrar.LRAR_ERR_INVALID  # overlap
    assert L.lrar_copy(FAKE, FAKE * 2, 0, None) == lrar.LRAR_OK


def test_read_stream_rejects(L):
    sink_bytes = L.lrar_read_stream_sink_bytes()
    assert sink_bytes > 0 and sink_bytes % 4 == 0
    assert L.lrar_read_stream(FAKE + 8, 64, FAKE * 4, None) == lrar.LRAR_ERR_INVALID
    assert L.lrar_read_stream(FAKE, 60, FAKE * 4, None) == lrar.LRAR_ERR_INVALID
    assert L.lrar_read_stream(FAKE, 64, None, None) == lrar.LRAR_ERR_INVALID
    assert L.lrar_read_stream(FAKE, 64, FAKE * 4 + 2, None) == lrar.LRAR_ERR_INVALID
    assert L.lrar_read_stream(FAKE, 64, FAKE + 32, None) == lrar.LRAR_ERR_INVALID  # overlap
    assert L.lrar_read_stream(FAKE, 0, None, None) == lrar.LRAR_OK


def mix(L, T=4, d=8, n=2, ld=8, out=FAKE * 2, out_ld=8, waves=8, depth=1, slots=4, rows=4,
        ptr=FAKE, odt=lrar.LRAR_BF16, nout=None, table=True, lock=0, wpr=1):
    """lrar_mix_stream through ctypes; out and out_ld may be one value or a list per output."""
    p = (ctypes.c_void_p * max(n, 1))(*([ptr] * max(n, 1)))
    l = (ctypes.c_int64 * max(n, 1))(*([ld] * max(n, 1)))
    outs = out if isinstance(out, list) else [out]
    lds = out_ld if isinstance(out_ld, list) else [out_ld] * len(outs)
    o = (ctypes.c_void_p * len(outs))(*outs)
    ol = (ctypes.c_int64 * len(outs))(*lds)
    k = len(outs) if nout is None else nout
    return L.lrar_mix_stream(T, d, n, p, l, k, o if table else None, ol if table else None, odt,
                             waves, wpr, depth, slots, rows, lock, None)


@pytest.mark.parametrize("kw", [
    dict(T=-1), dict(d=0), dict(d=12, ld=16, out_ld=16), dict(n=0), dict(n=65), dict(ld=4),
    dict(ld=12, d=8), dict(ptr=FAKE + 8), dict(out=None), dict(out_ld=4), dict(out=FAKE * 2 + 8),
    dict(out_ld=12), dict(waves=0), dict(waves=3), dict(waves=36), dict(depth=0), dict(depth=3),
    dict(depth=8), dict(rows=-1), dict(out=FAKE), dict(out=FAKE + 16, T=4), dict(slots=0),
    dict(slots=3), dict(slots=32), dict(slots=16, depth=2), dict(slots=8, depth=4),
    dict(nout=0), dict(nout=65), dict(odt=2), dict(table=False),
    dict(odt=lrar.LRAR_F32, out_ld=10),                         # 40-byte rows: not in 16s
    dict(odt=lrar.LRAR_F32, d=16, ld=16, out_ld=18),            # 72-byte rows: not in 16s
    dict(out=[FAKE * 2, FAKE * 2 + 16]),                        # two outputs overlap
    dict(out=[FAKE * 2, FAKE * 3], odt=lrar.LRAR_F32, out_ld=[8, 8], T=4,
         ptr=FAKE * 3 + 16),                                    # an output overlaps a source
    dict(out=[FAKE * 2, None]), dict(lock=-1), dict(lock=3), dict(wpr=0), dict(wpr=3),
    dict(wpr=8),
])
def test_mix_stream_rejects(L, kw):
    assert mix(L, **kw) == lrar.LRAR_ERR_INVALID, kw


def test_mix_stream_empty_is_ok(L):
    assert mix(L, T=0) == lrar.LRAR_OK
    assert mix(L, T=0, odt=lrar.LRAR_F32, out_ld=12) == lrar.LRAR_OK
    assert mix(L, T=0, out=None) == lrar.LRAR_OK
    assert mix(L, T=0, table=False) == lrar.LRAR_OK
    assert mix(L, T=0, lock=2) == lrar.LRAR_OK
    assert mix(L, T=0, wpr=4, lock=1) == lrar.LRAR_OK


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    monkeypatch.setattr(lrar, "LIB_PATH", str(tmp_path / "absent.so"))
    monkeypatch.setattr(lrar, "_lib", None)
    with pytest.raises(lrar.LibraryNotBuilt):
        lrar.lib()


def test_row_strides_of_256_mib_are_unsupported(L):
    """The read kernels address a tile's rows by 32-bit byte offsets: a row stride above 256 MiB
    is refused before any device work (T = 0 keeps the call host-only)."""
    most = 1 << 27  # bf16 elements: 256 MiB, the largest stride taken
    assert fwd(L, T=0, ld=most) == lrar.LRAR_OK
    assert fwd(L, T=0, ld=most + 8) == lrar.LRAR_ERR_UNSUPPORTED
    assert "row stride" in L.lrar_last_error().decode()
    assert merge_acc(L, T=0, o_ld=most + 8) == lrar.LRAR_ERR_UNSUPPORTED
    assert merge_acc(L, T=0, b_ld=most + 8) == lrar.LRAR_ERR_UNSUPPORTED
    assert merge_acc(L, T=0, acc_ld=most // 2 + 8) == lrar.LRAR_ERR_UNSUPPORTED  # fp32 acc


def bwd_noalloc(L, T=4, d=8, r=4, n=2, dsrc=None, dq=FAKE * 8, dout=FAKE * 7, ld=8):
    p, lds_ = _src(n, ld)
    dsrc = dsrc if dsrc is not None else [FAKE * (10 + i) for i in range(n)]
    dp = (ctypes.c_void_p * n)(*dsrc)
    dl = (ctypes.c_int64 * n)(*([ld] * n))
    return L.lrar_backward_noalloc(T, d, r, 1e-6, 1, n, p, lds_, FAKE * 2, 0, dout, ld, dp, dl, 0,
                                   dq, None)


def test_backward_noalloc_checks_before_device_work(L):
    """The no-allocation backward validates like lrar_backward_grad and refuses a key whose
    query-gradient partials would not fit its scratch, all before touching the device."""
    assert bwd_noalloc(L, T=0) == lrar.LRAR_OK
    assert bwd_noalloc(L, dsrc=[FAKE * 10, FAKE * 10 + 64]) == lrar.LRAR_ERR_INVALID
    assert bwd_noalloc(L, dq=None) == lrar.LRAR_ERR_INVALID
    # d = r = 16384 over 2048 rows: at least 256 workgroups' partials, more than 32 MiB
    big = 16384
    assert bwd_noalloc(L, T=2048, d=big, r=big, n=1, ld=big, dsrc=[FAKE * 5000],
                       dout=FAKE * 9000, dq=FAKE * 20000) == lrar.LRAR_ERR_UNSUPPORTED
    assert "scratch" in L.lrar_last_error().decode()


def fwd_save(L, T=4, d=8, r=4, n=2, ld=8, out=FAKE * 2, saved=FAKE * 30, saved_ld=4):
    p, l = _src(n, ld)
    return L.lrar_forward_save(T, d, r, 1e-6, 1, n, p, l, FAKE * 3, out, 8, saved, saved_ld, 0,
                               None)


def bwd_saved(L, T=4, d=8, r=4, n=2, saved=FAKE * 30, saved_ld=4, dsrc=None):
    p, ld = _src(n, 8)
    dsrc = dsrc if dsrc is not None else [FAKE * (10 + i) for i in range(n)]
    dp = (ctypes.c_void_p * n)(*dsrc)
    dl = (ctypes.c_int64 * n)(*([8] * n))
    return L.lrar_backward_saved(T, d, r, 1, n, p, ld, FAKE * 2, saved, saved_ld, 0, FAKE * 7, 8,
                                 dp, dl, 0, FAKE * 8, FAKE * 9, 1 << 30, None)


@pytest.mark.parametrize("kw,what", [
    (dict(saved=None), "saved is null"), (dict(saved_ld=3), "saved_ld"),
    (dict(saved=FAKE * 2 + 8), "saved overlaps out"), (dict(saved=FAKE + 8), "saved overlaps src"),
])
def test_forward_save_rejects(L, kw, what):
    assert fwd_save(L, **kw) == lrar.LRAR_ERR_INVALID
    assert what in L.lrar_last_error().decode()


@pytest.mark.parametrize("kw,what", [
    (dict(saved=None), "saved is null"), (dict(saved_ld=3), "saved_ld"),
    (dict(dsrc=[FAKE * 30 + 16, FAKE * 11]), "dsrc[0] overlaps saved"),
])
def test_backward_saved_rejects(L, kw, what):
    assert bwd_saved(L, **kw) == lrar.LRAR_ERR_INVALID
    assert what in L.lrar_last_error().decode()


def test_saved_entry_points_empty(L):
    assert fwd_save(L, T=0, saved=None) == lrar.LRAR_OK
    assert bwd_saved(L, T=0, saved=None) == lrar.LRAR_OK
