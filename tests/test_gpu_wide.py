"""Rows that no register tile holds, on every entry point, against the oracle element by element:
vector rows past the widest tile (bf16 d > 16384, fp32 d > 8192) and element-path rows (odd
row strides or unaligned widths) past 2048 columns, at the widths of the LR-AttnRes paper's
matched models (App. I, "Matched model comparison": d = 2560) with its unaligned shapes and
strided sources (App. I, "Numerical correctness"). These run the column-chunked read and merge
(k_read_two_pass in its three key modes), the row-add kernel of the fused update, and the
one-wave-per-row backward (k_backward)."""
import numpy as np
import pytest
import torch

import oracle
import parity
import transformer_depth_wise_lrar_amd as lrar
from gpu_util import f64, io_of, needs_gpu, query, say, sources
from transformer_depth_wise_lrar_amd import synth

pytestmark = [pytest.mark.gpu, needs_gpu]

BITS = {"bf16": 8, "f32": 24}

# (d, r, io, row stride of the sources or None): past the widest vector tile, and element-path
# rows (odd strides, unaligned widths) past 2048 columns
WIDE = [
    (16392, 64, "bf16", None),
    (16392, 16392, "bf16", None),
    (8196, 100, "f32", None),
    (8196, 8196, "f32", None),
    (2560, 640, "bf16", 2561),
    (2560, 2560, "bf16", 2561),
    (2560, 64, "f32", 2563),
    (4097, 1024, "bf16", None),
    (4097, 4097, "f32", None),
]
IDS = [f"d{d}-r{r}-{io}-ld{ld}" for d, r, io, ld in WIDE]


def wide_sources(n, T, d, io, ld, seed):
    return sources(n, T, d, io, seed=seed, scale=(0.5, 4.0), row_stride=ld)


def check_read(srcs, q, r, eps, variant, where):
    say(f"[wide read] {where} variant={variant} T={srcs[0].shape[0]} d={srcs[0].shape[1]} r={r} "
        f"n={len(srcs)} io={io_of(srcs[0])} ld={srcs[0].stride(0)}")
    out, alpha = lrar.lrar_forward(srcs, q, r, eps, alpha=True, variant=variant)
    torch.cuda.synchronize()
    s64 = [f64(s) for s in srcs]
    h_ref, a_ref = oracle.forward(s64, f64(q), r, eps)
    parity.assert_weights(f64(alpha), a_ref, where + " alpha")
    parity.assert_read(f64(out), h_ref, a_ref, s64, io_of(srcs[0]), where + " h")
    return out


@pytest.mark.parametrize("d,r,io,ld", WIDE, ids=IDS)
@pytest.mark.parametrize("n", [1, 3, 10])
def test_wide_forward(d, r, io, ld, n):
    """lrar_forward auto and two-pass: the column-chunked kernel; a single source is the
    identity; the online variant, which holds a row in registers, is refused at T > 0."""
    srcs = wide_sources(n, 9, d, io, ld, seed=1000 + d + n)
    q = query(r, seed=1001)
    for variant in ("auto", "two_pass"):
        out = check_read(srcs, q, r, 1e-6, variant, f"d{d} r{r}")
        if n == 1:
            assert torch.equal(out, srcs[0])
    with pytest.raises(lrar.LrarError) as e:
        lrar.lrar_forward(srcs, q, r, 1e-6, variant="online")
    assert e.value.status == lrar.LRAR_ERR_UNSUPPORTED


def merge_case(d, r, io, ld, n_inter, n_extra, acc_dtype, seed, T=7):
    inter = wide_sources(n_inter, T, d, io, ld, seed)
    extra = wide_sources(n_extra, T, d, io, ld, seed + 1) if n_extra else []
    q = query(r, seed=seed + 2)
    s64 = [f64(s) for s in inter]
    m_o, l_o, acc_o = oracle.stats(s64, f64(q)[None, :], r, 1e-6)
    m = torch.tensor(m_o[0], dtype=torch.float32, device="cuda")
    l = torch.tensor(l_o[0], dtype=torch.float32, device="cuda")
    acc = torch.tensor(acc_o[0], dtype=torch.float32).to(acc_dtype).cuda()
    say(f"[wide merge] d={d} r={r} io={io} ld={ld} n_extra={n_extra} acc={acc_dtype}")
    out_dtype = torch.bfloat16 if io == "bf16" else torch.float32
    out, m2, l2 = lrar.lrar_merge(m, l, acc, extra, q, r, 1e-6, stats_out=True,
                                  io_dtype=out_dtype)
    torch.cuda.synchronize()
    e64 = [f64(s) for s in extra]
    m_in, l_in, acc_in = f64(m), f64(l), f64(acc)
    h_ref, m_ref, l_ref = oracle.merge(m_in, l_in, acc_in, e64, f64(q), r, 1e-6)
    if e64:
        z_e, _ = oracle.scores(e64, f64(q), r, 1e-6)
        w_extra = np.exp(z_e - m_ref[:, None]) / l_ref[:, None]
    else:
        w_extra = np.zeros((T, 0))
    w_prior = l_in * np.exp(m_in - m_ref) / l_ref
    parity.assert_merge(f64(out), h_ref, w_prior, acc_in / l_in[:, None], w_extra, e64, io,
                        "wide merge h")
    m2g = f64(m2)
    assert np.all(np.abs(m2g - m_ref) <= 2.0 ** -23 * np.abs(m_ref) + 1e-12)
    l_resc = l_ref * np.exp(m_ref - m2g)
    assert np.all(np.abs(f64(l2) - l_resc) <= 4 * parity.U * l_resc)


@pytest.mark.parametrize("d,r,io,ld", WIDE, ids=IDS)
@pytest.mark.parametrize("n_extra", [0, 1, 3])
@pytest.mark.parametrize("acc_dtype", [torch.float32, torch.bfloat16])
def test_wide_merge(d, r, io, ld, n_extra, acc_dtype):
    """lrar_merge on the column-chunked kernel (its merge instantiations, fp32 and bf16
    Phase-1 accumulators)."""
    merge_case(d, r, io, ld, 3, n_extra, acc_dtype, seed=1100 + d)


@pytest.mark.parametrize("d,r,io,ld", WIDE, ids=IDS)
def test_wide_fullrms(d, r, io, ld):
    """lrar_forward_fullrms on the column-chunked kernel: the key pass sums the square of every
    column of the row."""
    srcs = wide_sources(5, 7, d, io, ld, seed=1200 + d)
    q = query(r, seed=1201)
    say(f"[wide fullrms] d={d} r={r} io={io} ld={ld}")
    out, alpha = lrar.lrar_forward_fullrms(srcs, q, r, 1e-6, alpha=True)
    torch.cuda.synchronize()
    s64 = [f64(s) for s in srcs]
    h_ref, a_ref = oracle.forward_fullrms(s64, f64(q), r, 1e-6)
    parity.assert_weights(f64(alpha), a_ref, "wide fullrms alpha")
    parity.assert_read(f64(out), h_ref, a_ref, s64, io, "wide fullrms h")


def key_tensors(n, T, r, io, seed, offset=0):
    full = synth.values(n, T, r + offset + 1, io, seed, scale=(0.5, 2.0), device="cuda")
    return [x[:, offset:offset + r] for x in full]


@pytest.mark.parametrize("d,r,io,ld,koff", [
    (16392, 64, "bf16", None, 0), (8196, 100, "f32", None, 1), (2560, 640, "bf16", 2561, 0),
    (4097, 1024, "bf16", None, 3),
    # rows that fit a tile, keys that no spread piece serves: r > 512, or misaligned pieces
    (1024, 1000, "bf16", None, 0), (2048, 768, "f32", None, 0), (1024, 96, "bf16", None, 1),
])
def test_wide_keys(d, r, io, ld, koff):
    """lrar_forward_keys on the column-chunked kernel: the key pass reads each source's key
    row element by element (any alignment, any r)."""
    srcs = wide_sources(4, 7, d, io, ld, seed=1300 + d)
    keys = key_tensors(4, 7, r, io, seed=1301, offset=koff)
    q = query(r, seed=1302)
    say(f"[wide keys] d={d} r={r} io={io} ld={ld} key offset={koff}")
    out, alpha = lrar.lrar_forward_keys(srcs, keys, q, r, 1e-6, alpha=True)
    torch.cuda.synchronize()
    s64 = [f64(s) for s in srcs]
    h_ref, a_ref = oracle.forward_keys(s64, [f64(k) for k in keys], f64(q), r, 1e-6)
    parity.assert_weights(f64(alpha), a_ref, "wide keys alpha")
    parity.assert_read(f64(out), h_ref, a_ref, s64, io, "wide keys h")


@pytest.mark.parametrize("d,r,io,ld", WIDE, ids=IDS)
@pytest.mark.parametrize("with_b,in_place", [(True, False), (True, True), (False, False)])
def test_wide_merge_accumulate(d, r, io, ld, with_b, in_place):
    """lrar_merge_accumulate on rows past a tile: the row-add kernel writes b' = b + o (bit for
    bit the oracle's rounding), then the column-chunked merge reads b'."""
    T = 7
    inter = wide_sources(3, T, d, io, ld, seed=1400 + d)
    b, o = wide_sources(2, T, d, io, ld, seed=1401 + d)
    q = query(r, seed=1402)
    s64 = [f64(s) for s in inter]
    m_o, l_o, acc_o = oracle.stats(s64, f64(q)[None, :], r, 1e-6)
    m = torch.tensor(m_o[0], dtype=torch.float32, device="cuda")
    l = torch.tensor(l_o[0], dtype=torch.float32, device="cuda")
    acc = torch.tensor(acc_o[0], dtype=torch.float32).cuda()
    b64 = f64(b) if with_b else None
    o64 = f64(o)
    say(f"[wide merge_acc] d={d} r={r} io={io} ld={ld} b={with_b} in_place={in_place}")
    out, b2, m2, l2 = lrar.lrar_merge_accumulate(m, l, acc, b if with_b else None, o, q, r, 1e-6,
                                                 b_out=b if in_place else None, stats_out=True)
    torch.cuda.synchronize()
    m_in, l_in, acc_in = f64(m), f64(l), f64(acc)
    h_ref, bref, m_ref, l_ref = oracle.merge_accumulate(m_in, l_in, acc_in, b64, o64, f64(q), r,
                                                        1e-6, BITS[io])
    assert np.array_equal(f64(b2), bref), "b_out differs from round(b + o)"
    z_e, _ = oracle.scores([bref], f64(q), r, 1e-6)
    w_extra = np.exp(z_e - m_ref[:, None]) / l_ref[:, None]
    w_prior = l_in * np.exp(m_in - m_ref) / l_ref
    parity.assert_merge(f64(out), h_ref, w_prior, acc_in / l_in[:, None], w_extra, [bref], io,
                        "wide merge_acc h")
    assert np.all(np.abs(f64(m2) - m_ref) <= 2.0 ** -23 * np.abs(m_ref) + 1e-12)


@pytest.mark.parametrize("d,r,io,ld", [
    (2560, 640, "bf16", 2561), (2560, 2560, "bf16", 2561), (2560, 64, "f32", 2563),
    (4097, 1024, "bf16", None), (3000, 3000, "f32", None),
    (16392, 64, "bf16", None), (16384, 64, "f32", None), (20000, 2000, "bf16", None),
])
@pytest.mark.parametrize("grad", ["f32", "bf16"])
@pytest.mark.parametrize("accumulate", [False, True])
def test_wide_backward(d, r, io, ld, grad, accumulate):
    """The one-wave-per-row backward on element-path rows past 2048 columns and on vector rows
    past the widest row tile, with fp32 and bf16 gradients, with and without accumulation."""
    T, n = 9, 4
    srcs = wide_sources(n, T, d, io, ld, seed=1500 + d)
    q = query(r, seed=1501)
    gdt = torch.float32 if grad == "f32" else torch.bfloat16
    dout = synth.upstream(T, d, 1502, device="cpu").to(gdt).cuda()
    prior = dsrc = None
    if accumulate:
        prior = [torch.randn((T, d), generator=torch.Generator().manual_seed(1503 + i))
                 .to(gdt).cuda() for i in range(n)]
        dsrc = [p.clone() for p in prior]
    say(f"[wide backward] d={d} r={r} io={io} ld={ld} grad={grad} accumulate={accumulate}")
    dsrc, dq = lrar.lrar_backward_grad(srcs, q, dout, r, 1e-6, dsrc=dsrc, accumulate=accumulate)
    torch.cuda.synchronize()
    s64 = [f64(s) for s in srcs]
    g64 = f64(dout)
    ds_ref, dq_ref = oracle.backward(s64, f64(q), g64, r, 1e-6)
    for i in range(n):
        ref = ds_ref[i] + (f64(prior[i]) if accumulate else 0.0)
        if grad == "f32":
            parity.assert_dsrc(f64(dsrc[i]), ref, f"wide dsrc[{i}]")
        else:
            parity.assert_dsrc_bf16(f64(dsrc[i]), ref, f"wide dsrc[{i}]")
    h, al = oracle.forward(s64, f64(q), r, 1e-6)
    parity.assert_dq(f64(dq), dq_ref, parity.dq_bound(s64, f64(q), g64, al, h, r, 1e-6),
                     "wide dq")


def test_wide_backward_key_too_wide_is_refused():
    """An element-path key spanning more than 64 chunks of 64 columns is refused at T > 0."""
    srcs = wide_sources(2, 3, 8192, "bf16", 8193, seed=1600)
    q = query(8192, seed=1601)
    dout = torch.zeros((3, 8192), dtype=torch.float32, device="cuda")
    with pytest.raises(lrar.LrarError) as e:
        lrar.lrar_backward(srcs, q, dout, 8192, 1e-6)
    assert e.value.status == lrar.LRAR_ERR_UNSUPPORTED


@pytest.mark.parametrize("io", ["bf16", "f32"])
def test_column_slices_of_one_buffer(io):
    """Sources and the output as column slices of one [T, 4d] buffer share its row stride and
    interleave without overlapping: the byte-range check accepts them and the read is exact.
    An output slice that overlaps a source's columns is refused."""
    T, d, r = 37, 1024, 64
    dt = torch.bfloat16 if io == "bf16" else torch.float32
    buf = torch.randn((T, 4 * d), generator=torch.Generator().manual_seed(1700)).to(dt).cuda()
    srcs = [buf[:, 0:d], buf[:, d:2 * d], buf[:, 2 * d:3 * d]]
    out = buf[:, 3 * d:4 * d]
    q = query(r, seed=1701)
    s64 = [f64(s) for s in srcs]  # before the call: out shares the buffer
    say(f"[column slices] io={io}")
    lrar.lrar_forward(srcs, q, r, 1e-6, out=out)
    torch.cuda.synchronize()
    h_ref, a_ref = oracle.forward(s64, f64(q), r, 1e-6)
    parity.assert_read(f64(out), h_ref, a_ref, s64, io, "column slices h")
    assert np.array_equal(f64(buf[:, :3 * d]), np.concatenate(s64, axis=1))
    with pytest.raises(lrar.LrarError) as e:
        lrar.lrar_forward(srcs, q, r, 1e-6, out=buf[:, 2 * d + 8:3 * d + 8])
    assert e.value.status == lrar.LRAR_ERR_INVALID
