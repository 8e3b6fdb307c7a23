"""Seeded random shapes across the dispatch boundaries of every entry point (the read, Phase 1,
the merge, the fused update, the full-width-RMS and separate-key reads, and the backward),
against the oracle element by element. The widths straddle the register-tile limits (one to four chunks of 64
units per wave, rows shared by two or four waves, rows past the widest tile), the key widths map to
every spread-piece size, to the row units and to keys that start inside a unit, unaligned widths
and odd row strides take the element path, and every case draws its element type, 1 to 20
sources and 1 to 300 rows (ragged tiles); Phase 1 also draws 1 to 20 site queries and the
accumulators' type and row padding, the merges their prior sources and extra sources."""
import numpy as np
import pytest
import torch

import oracle
import parity
import transformer_depth_wise_lrar_amd as lrar
from gpu_util import f64, needs_gpu, query, say, sources
from transformer_depth_wise_lrar_amd import synth

pytestmark = [pytest.mark.gpu, needs_gpu]

WIDTHS = [8, 16, 64, 72, 513, 512, 520, 1001, 1024, 1032, 1536, 2048, 2056, 3000, 4096, 4104,
          7168, 8192, 8200]
ROWS = [1, 3, 37, 130, 300]


def draw(rng, widths):
    d = int(rng.choice(widths))
    io = str(rng.choice(["bf16", "f32"]))
    keys = [1, 8, 16, 32, 33, 64, 100, 128, 256, 257, 512, d // 4, d // 2, d - 1, d]
    r = int(rng.choice([k for k in keys if 1 <= k <= d]))
    n = int(rng.integers(1, 21))
    T = int(rng.choice(ROWS))
    ld = rng.choice([None, d + 8, d + 1])
    return d, r, io, n, T, (None if ld is None else int(ld))


def cases(seed, count, widths):
    rng = np.random.default_rng(seed)
    return [draw(rng, widths) for _ in range(count)]


FWD = cases(7001, 48, WIDTHS)
# the backward serves keys past a register tile only up to a window of chunks: widths that a
# row tile holds, and element-path rows up to 3000 columns
BWD = cases(7002, 24, [w for w in WIDTHS if w <= 4104 or w in (7168, 8192)])


def ids(cs):
    return [f"d{d}-r{r}-{io}-n{n}-T{T}-ld{ld}" for d, r, io, n, T, ld in cs]


@pytest.mark.parametrize("d,r,io,n,T,ld", FWD, ids=ids(FWD))
def test_random_forward(d, r, io, n, T, ld):
    eps = 1e-6
    srcs = sources(n, T, d, io, seed=d + 7 * r + n, scale=(0.5, 4.0), row_stride=ld)
    q = query(r, seed=r + 11)
    s64 = [f64(s) for s in srcs]
    h_ref, a_ref = oracle.forward(s64, f64(q), r, eps)
    for variant in ("auto", "two_pass"):
        say(f"[random] forward d={d} r={r} io={io} n={n} T={T} ld={ld} {variant}")
        out, alpha = lrar.lrar_forward(srcs, q, r, eps, alpha=True, variant=variant)
        torch.cuda.synchronize()
        where = f"d={d} r={r} {io} n={n} T={T} ld={ld} {variant}"
        parity.assert_weights(f64(alpha), a_ref, where + " alpha")
        parity.assert_read(f64(out), h_ref, a_ref, s64, io, where + " h")
    say(f"[random] forward_save d={d} r={r} io={io} n={n} T={T} ld={ld}")
    out, saved = lrar.lrar_forward_save(srcs, q, r, eps)
    torch.cuda.synchronize()
    z_o, rho_o = oracle.scores(s64, f64(q), r, eps)
    sv = f64(saved)
    assert np.all(np.abs(sv[:, :n] - z_o) <= 1e-12 * np.maximum(1.0, np.abs(z_o)) + 1e-12)
    assert np.all(np.abs(sv[:, n:2 * n] * rho_o - 1.0) <= 1e-13)
    parity.assert_read(f64(out), h_ref, a_ref, s64, io, f"d={d} r={r} save h")


@pytest.mark.parametrize("d,r,io,n,T,ld", BWD, ids=ids(BWD))
def test_random_backward(d, r, io, n, T, ld):
    eps = 1e-6
    srcs = sources(n, T, d, io, seed=d + 3 * r + n, scale=(0.5, 4.0), row_stride=ld)
    q = query(r, seed=r + 13)
    dout = synth.upstream(T, d, d + r, device="cpu").cuda()
    say(f"[random] backward d={d} r={r} io={io} n={n} T={T} ld={ld}")
    dsrc, dq = lrar.lrar_backward(srcs, q, dout, r, eps)
    torch.cuda.synchronize()
    s64 = [f64(s) for s in srcs]
    g64 = f64(dout)
    ds_ref, dq_ref = oracle.backward(s64, f64(q), g64, r, eps)
    where = f"d={d} r={r} {io} n={n} T={T} ld={ld}"
    for i in range(n):
        parity.assert_dsrc(f64(dsrc[i]), ds_ref[i], f"{where} dsrc[{i}]")
    h, al = oracle.forward(s64, f64(q), r, eps)
    parity.assert_dq(f64(dq), dq_ref, parity.dq_bound(s64, f64(q), g64, al, h, r, eps),
                     f"{where} dq")


def draw_keyed(rng):
    d, r, io, n, T, ld = draw(rng, WIDTHS)
    return d, r, io, n, T, ld, int(rng.integers(0, 1 << 30))


STATS = [draw_keyed(np.random.default_rng(7003 + i)) for i in range(20)]
MERGE = [draw_keyed(np.random.default_rng(7103 + i)) for i in range(16)]
MACC = [draw_keyed(np.random.default_rng(7203 + i)) for i in range(16)]
FULL = cases(7004, 16, WIDTHS)
KEYS = [draw_keyed(np.random.default_rng(7303 + i)) for i in range(16)]


def kids(cs):
    return [f"d{d}-r{r}-{io}-n{n}-T{T}-ld{ld}-k{k % 1000}" for d, r, io, n, T, ld, k in cs]


def stats_rounded(inter64, q64, r, eps, acc_dtype):
    """The oracle's Phase-1 statistics of one query, rounded to their storage types."""
    m_o, l_o, acc_o = oracle.stats(inter64, q64[None, :], r, eps)
    m = torch.tensor(m_o[0], dtype=torch.float32, device="cuda")
    l = torch.tensor(l_o[0], dtype=torch.float32, device="cuda")
    acc = torch.tensor(acc_o[0], dtype=torch.float32).to(acc_dtype).cuda()
    return m, l, acc


@pytest.mark.parametrize("d,r,io,n,T,ld,k", STATS, ids=kids(STATS))
def test_random_stats(d, r, io, n, T, ld, k):
    rng = np.random.default_rng(k)
    nq = int(rng.integers(1, 21))
    n = min(n, 12)
    acc_dtype = torch.bfloat16 if rng.integers(0, 2) else torch.float32
    pad = int(rng.choice([0, 8]))
    eps = 1e-6
    srcs = sources(n, T, d, io, seed=k % 9973, scale=(0.5, 4.0), row_stride=ld)
    qs = query(r, seed=k % 997, nq=nq)
    acc = torch.full((nq, T, d + pad), float("nan"), dtype=acc_dtype, device="cuda")[:, :, :d]
    m = torch.empty((nq, T), dtype=torch.float32, device="cuda")
    l = torch.empty((nq, T), dtype=torch.float32, device="cuda")
    where = f"d={d} r={r} {io} n={n} nq={nq} T={T} ld={ld} acc={acc_dtype} pad={pad}"
    say(f"[random] stats {where}")
    lrar.lrar_forward_stats(srcs, qs, r, eps, m=m, l=l, acc=acc)
    torch.cuda.synchronize()
    s64 = [f64(s) for s in srcs]
    q64 = f64(qs)
    m_o, l_o, acc_o = oracle.stats(s64, q64, r, eps)
    m_g, l_g, acc_g = f64(m), f64(l), f64(acc)
    for qi in range(nq):
        z_o, _ = oracle.scores(s64, q64[qi], r, eps)
        parity.assert_stats(m_g[qi], l_g[qi], acc_g[qi], m_o[qi], l_o[qi], acc_o[qi], z_o, s64,
                            "bf16" if acc_dtype == torch.bfloat16 else "f32",
                            f"{where} query {qi}")


@pytest.mark.parametrize("d,r,io,n,T,ld,k", MERGE, ids=kids(MERGE))
def test_random_merge(d, r, io, n, T, ld, k):
    rng = np.random.default_rng(k)
    n_inter = int(rng.integers(1, 9))
    n_extra = int(rng.integers(0, 4))
    acc_dtype = torch.bfloat16 if rng.integers(0, 2) else torch.float32
    eps = 1e-6
    inter = sources(n_inter, T, d, io, seed=k % 9973, scale=(0.5, 4.0))
    extra = (sources(n_extra, T, d, io, seed=k % 9967, scale=(0.5, 4.0), row_stride=ld)
             if n_extra else [])
    q = query(r, seed=k % 991)
    m, l, acc = stats_rounded([f64(s) for s in inter], f64(q), r, eps, acc_dtype)
    where = f"d={d} r={r} {io} inter={n_inter} extra={n_extra} T={T} ld={ld} acc={acc_dtype}"
    say(f"[random] merge {where}")
    out_dtype = torch.bfloat16 if io == "bf16" else torch.float32
    out, m2, l2 = lrar.lrar_merge(m, l, acc, extra, q, r, eps, stats_out=True, io_dtype=out_dtype)
    torch.cuda.synchronize()
    e64 = [f64(s) for s in extra]
    m_in, l_in, acc_in = f64(m), f64(l), f64(acc)
    h_ref, m_ref, l_ref = oracle.merge(m_in, l_in, acc_in, e64, f64(q), r, eps)
    if e64:
        z_e, _ = oracle.scores(e64, f64(q), r, eps)
        w_extra = np.exp(z_e - m_ref[:, None]) / l_ref[:, None]
    else:
        w_extra = np.zeros((T, 0))
    w_prior = l_in * np.exp(m_in - m_ref) / l_ref
    parity.assert_merge(f64(out), h_ref, w_prior, acc_in / l_in[:, None], w_extra, e64, io,
                        where + " h")
    m2g = f64(m2)
    assert np.all(np.abs(m2g - m_ref) <= 2.0 ** -23 * np.abs(m_ref) + 1e-12), where + " m'"
    l_resc = l_ref * np.exp(m_ref - m2g)
    assert np.all(np.abs(f64(l2) - l_resc) <= 4 * parity.U * l_resc), where + " l'"


@pytest.mark.parametrize("d,r,io,n,T,ld,k", MACC, ids=kids(MACC))
def test_random_merge_accumulate(d, r, io, n, T, ld, k):
    rng = np.random.default_rng(k)
    n_inter = int(rng.integers(1, 9))
    with_b = bool(rng.integers(0, 2))
    acc_dtype = torch.bfloat16 if rng.integers(0, 2) else torch.float32
    eps = 1e-6
    inter = sources(n_inter, T, d, io, seed=k % 9973, scale=(0.5, 4.0))
    b, o = sources(2, T, d, io, seed=k % 9967, scale=(0.5, 4.0), row_stride=ld)
    q = query(r, seed=k % 991)
    m, l, acc = stats_rounded([f64(s) for s in inter], f64(q), r, eps, acc_dtype)
    where = f"d={d} r={r} {io} inter={n_inter} b={with_b} T={T} ld={ld} acc={acc_dtype}"
    say(f"[random] merge_accumulate {where}")
    out, b2, m2, l2 = lrar.lrar_merge_accumulate(m, l, acc, b if with_b else None, o, q, r, eps,
                                                 stats_out=True)
    torch.cuda.synchronize()
    m_in, l_in, acc_in = f64(m), f64(l), f64(acc)
    h_ref, bref, m_ref, l_ref = oracle.merge_accumulate(
        m_in, l_in, acc_in, f64(b) if with_b else None, f64(o), f64(q), r, eps,
        8 if io == "bf16" else 24)
    assert np.array_equal(f64(b2), bref), where + " b_out differs from round(b + o)"
    z_e, _ = oracle.scores([bref], f64(q), r, eps)
    w_extra = np.exp(z_e - m_ref[:, None]) / l_ref[:, None]
    w_prior = l_in * np.exp(m_in - m_ref) / l_ref
    parity.assert_merge(f64(out), h_ref, w_prior, acc_in / l_in[:, None], w_extra, [bref], io,
                        where + " h")
    m2g = f64(m2)
    assert np.all(np.abs(m2g - m_ref) <= 2.0 ** -23 * np.abs(m_ref) + 1e-12), where + " m'"
    l_resc = l_ref * np.exp(m_ref - m2g)
    assert np.all(np.abs(f64(l2) - l_resc) <= 4 * parity.U * l_resc), where + " l'"


@pytest.mark.parametrize("d,r,io,n,T,ld", FULL, ids=ids(FULL))
def test_random_fullrms(d, r, io, n, T, ld):
    eps = 1e-6
    srcs = sources(n, T, d, io, seed=d + 5 * r + n, scale=(0.5, 4.0), row_stride=ld)
    q = query(r, seed=r + 17)
    where = f"d={d} r={r} {io} n={n} T={T} ld={ld}"
    say(f"[random] fullrms {where}")
    out, alpha = lrar.lrar_forward_fullrms(srcs, q, r, eps, alpha=True)
    torch.cuda.synchronize()
    s64 = [f64(s) for s in srcs]
    h_ref, a_ref = oracle.forward_fullrms(s64, f64(q), r, eps)
    parity.assert_weights(f64(alpha), a_ref, where + " alpha")
    parity.assert_read(f64(out), h_ref, a_ref, s64, io, where + " h")


@pytest.mark.parametrize("d,r,io,n,T,ld,k", KEYS, ids=kids(KEYS))
def test_random_keys(d, r, io, n, T, ld, k):
    rng = np.random.default_rng(k)
    key_pad = int(rng.choice([0, 8, 1]))
    eps = 1e-6
    srcs = sources(n, T, d, io, seed=k % 9973, scale=(0.5, 4.0), row_stride=ld)
    full = synth.values(n, T, r + key_pad, io, k % 9967, scale=(0.5, 2.0), device="cpu")
    keys = [x.cuda()[:, :r] for x in full]
    q = query(r, seed=k % 991)
    where = f"d={d} r={r} {io} n={n} T={T} ld={ld} key_ld={r + key_pad}"
    say(f"[random] keys {where}")
    out, alpha = lrar.lrar_forward_keys(srcs, keys, q, r, eps, alpha=True)
    torch.cuda.synchronize()
    s64 = [f64(s) for s in srcs]
    h_ref, a_ref = oracle.forward_keys(s64, [f64(x) for x in keys], f64(q), r, eps)
    parity.assert_weights(f64(alpha), a_ref, where + " alpha")
    parity.assert_read(f64(out), h_ref, a_ref, s64, io, where + " h")


BWD2 = [draw_keyed(np.random.default_rng(7403 + i)) for i in range(24)]
BWD2 = [c for c in BWD2 if c[0] <= 4104 or c[0] in (7168, 8192)]


@pytest.mark.parametrize("d,r,io,n,T,ld,k", BWD2, ids=kids(BWD2))
def test_random_backward_grad_saved(d, r, io, n, T, ld, k):
    """lrar_backward_grad (fp32 or bf16 gradients, with or without accumulation) and the same
    from lrar_forward_save's statistics (lrar_backward_saved), against the oracle."""
    rng = np.random.default_rng(k)
    grad = str(rng.choice(["f32", "bf16"]))
    accumulate = bool(rng.integers(0, 2))
    saved_stats = bool(rng.integers(0, 2))
    eps = 1e-6
    srcs = sources(n, T, d, io, seed=k % 9973, scale=(0.5, 4.0), row_stride=ld)
    q = query(r, seed=k % 991)
    gdt = torch.float32 if grad == "f32" else torch.bfloat16
    dout = synth.upstream(T, d, k % 9967, device="cpu").to(gdt).cuda()
    prior = dsrc = None
    if accumulate:
        prior = [torch.randn((T, d), generator=torch.Generator().manual_seed(k % 997 + i))
                 .to(gdt).cuda() for i in range(n)]
        dsrc = [p.clone() for p in prior]
    where = (f"d={d} r={r} {io} n={n} T={T} ld={ld} grad={grad} acc={accumulate} "
             f"saved={saved_stats}")
    say(f"[random] backward_grad {where}")
    if saved_stats:
        _, saved = lrar.lrar_forward_save(srcs, q, r, eps)
        dsrc, dq = lrar.lrar_backward_saved(srcs, q, saved, dout, r, dsrc=dsrc,
                                            accumulate=accumulate)
    else:
        dsrc, dq = lrar.lrar_backward_grad(srcs, q, dout, r, eps, dsrc=dsrc,
                                           accumulate=accumulate)
    torch.cuda.synchronize()
    s64 = [f64(s) for s in srcs]
    g64 = f64(dout)
    ds_ref, dq_ref = oracle.backward(s64, f64(q), g64, r, eps)
    for i in range(n):
        ref = ds_ref[i] + (f64(prior[i]) if accumulate else 0.0)
        if grad == "f32":
            parity.assert_dsrc(f64(dsrc[i]), ref, f"{where} dsrc[{i}]")
        else:
            parity.assert_dsrc_bf16(f64(dsrc[i]), ref, f"{where} dsrc[{i}]")
    h, al = oracle.forward(s64, f64(q), r, eps)
    parity.assert_dq(f64(dq), dq_ref, parity.dq_bound(s64, f64(q), g64, al, h, r, eps),
                     f"{where} dq")
