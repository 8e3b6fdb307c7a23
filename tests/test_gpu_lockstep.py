"""Reads whose waves meet at workgroup barriers (the lockstep of the one-wave rows through the
three-deep ring, once per ring cycle; of the shallower rings from 8 sources, once per tile; of
the four-wave rows with a spread key, once per tile; and of the fused Phase-2 update's one-wave
rows, once per tile), on row counts whose last step leaves
some row groups of a workgroup without a tile, where the barrier must be skipped by all of the
workgroup's waves alike.

Each test fills the output with NaN, then checks that every row was written, that every row's
weights sum to 1, and that sampled rows (the ends, the ragged tail and random rows) match the
oracle element by element.
"""
import numpy as np
import pytest
import torch

import oracle
import parity
import transformer_depth_wise_lrar_amd as lrar
from gpu_util import f64, needs_gpu, sample_rows, say
from transformer_depth_wise_lrar_amd import synth

pytestmark = [pytest.mark.gpu, needs_gpu]


def rows64(t, rows):
    idx = torch.as_tensor(rows, device=t.device)
    return f64(t.index_select(0, idx))


def check(out, alpha, T, rows, ref_fn, srcs, where):
    assert not torch.isnan(out.float()).any(), where + ": a row was not written"
    sums = alpha.double().sum(dim=1)
    assert torch.all((sums - 1.0).abs() < 1e-5), where + ": weights do not sum to 1"
    s64 = [rows64(s, rows) for s in srcs]
    h_ref, a_ref = ref_fn(s64)
    parity.assert_weights(rows64(alpha, rows), a_ref, where + " alpha")
    parity.assert_read(rows64(out, rows), h_ref, a_ref, s64, "bf16", where + " h")


@pytest.mark.parametrize("d,r,n,T", [
    (1024, 64, 20, 16384 + 37),    # three-deep ring: a barrier per ring cycle
    (1024, 64, 49, 16384 + 37),    # the same over 12 ring cycles a tile
    (1024, 64, 9, 16384 + 37),     # two-deep ring, 8+ sources: a barrier per tile
    (1024, 64, 7, 16384 + 37),     # below 8 sources: no barrier
    (2048, 64, 10, 65536 + 37),    # drained one ahead, one-wave rows: per tile, 8-tile launches
    (2048, 2048, 8, 65536 + 37),   # key from the row units of one wave: per tile
    (4096, 64, 10, 16384 + 37),    # four-wave rows with a spread key: per tile
])
def test_lockstep_reads(d, r, n, T):
    eps = 1e-6
    srcs = synth.values(n, T, d, "bf16", seed=950 + n, scale=(0.5, 4.0), device="cuda")
    q = synth.queries(1, r, 1.0, seed=951 + r, device="cuda")[0].contiguous()
    out = torch.full((T, d), float("nan"), dtype=torch.bfloat16, device="cuda")
    alpha = torch.full((T, n), float("nan"), dtype=torch.float32, device="cuda")
    where = f"lockstep d={d} r={r} n={n} T={T}"
    say(f"[lockstep] {where}")
    lrar.lrar_forward(srcs, q, r, eps, out=out, alpha=alpha, variant="online")
    torch.cuda.synchronize()
    rows = sample_rows(T, 40, seed=T + n)
    check(out, alpha, T, rows, lambda s64: oracle.forward(s64, f64(q), r, eps), srcs, where)


@pytest.mark.parametrize("n", [8, 20])
def test_lockstep_separate_keys(n):
    """The separate-key read takes the three-deep ring from 8 sources, with its per-cycle
    barrier."""
    T, d, r, eps = 16384 + 37, 1024, 32, 1e-6
    srcs = synth.values(n, T, d, "bf16", seed=960 + n, scale=(0.5, 4.0), device="cuda")
    keys = synth.values(n, T, r, "bf16", seed=961 + n, scale=(0.5, 2.0), device="cuda")
    q = synth.queries(1, r, 1.0, seed=962, device="cuda")[0].contiguous()
    out = torch.full((T, d), float("nan"), dtype=torch.bfloat16, device="cuda")
    alpha = torch.full((T, n), float("nan"), dtype=torch.float32, device="cuda")
    where = f"lockstep keys n={n} T={T}"
    say(f"[lockstep] {where}")
    lrar.lrar_forward_keys(srcs, keys, q, r, eps, out=out, alpha=alpha)
    torch.cuda.synchronize()
    rows = sample_rows(T, 40, seed=T + n)
    k64 = [rows64(k, rows) for k in keys]
    check(out, alpha, T, rows, lambda s64: oracle.forward_keys(s64, k64, f64(q), r, eps), srcs,
          where)


@pytest.mark.parametrize("acc_dtype", [torch.float32, torch.bfloat16])
def test_lockstep_fused_update(acc_dtype):
    """The fused Phase-2 update's one-wave rows meet once per tile: b' = b + o bit for bit and h
    within the merge's bar on sampled rows, every row written."""
    T, d, r, eps = 65536 + 37, 2048, 64, 1e-6
    b, o = synth.values(2, T, d, "bf16", seed=970, scale=(0.5, 4.0), device="cuda")
    q = synth.queries(1, r, 1.0, seed=971, device="cuda")[0].contiguous()
    g = torch.Generator(device="cuda").manual_seed(972)
    m = (10.0 + torch.randn((T,), generator=g, device="cuda")).float()
    l = (1.0 + torch.rand((T,), generator=g, device="cuda")).float()
    acc = torch.randn((T, d), generator=g, device="cuda").to(acc_dtype)
    out = torch.full((T, d), float("nan"), dtype=torch.bfloat16, device="cuda")
    b_out = torch.full((T, d), float("nan"), dtype=torch.bfloat16, device="cuda")
    where = f"lockstep fused update acc={acc_dtype} T={T}"
    say(f"[lockstep] {where}")
    lrar.lrar_merge_accumulate(m, l, acc, b, o, q, r, eps, out=out, b_out=b_out)
    torch.cuda.synchronize()
    assert not torch.isnan(out.float()).any(), where + ": a row of h was not written"
    assert not torch.isnan(b_out.float()).any(), where + ": a row of b' was not written"
    rows = sample_rows(T, 40, seed=T)
    m_in = rows64(m[:, None], rows)[:, 0]
    l_in = rows64(l[:, None], rows)[:, 0]
    acc_in = rows64(acc, rows)
    h_ref, bref, m_ref, l_ref = oracle.merge_accumulate(m_in, l_in, acc_in, rows64(b, rows),
                                                        rows64(o, rows), f64(q), r, eps, 8)
    assert np.array_equal(rows64(b_out, rows), bref), where + ": b' differs from round(b + o)"
    z_e, _ = oracle.scores([bref], f64(q), r, eps)
    w_extra = np.exp(z_e - m_ref[:, None]) / l_ref[:, None]
    w_prior = l_in * np.exp(m_in - m_ref) / l_ref
    parity.assert_merge(rows64(out, rows), h_ref, w_prior, acc_in / l_in[:, None], w_extra,
                        [bref], "bf16", where + " h")


@pytest.mark.parametrize("grad", ["f32", "bf16"])
def test_lockstep_backward_d1024(grad):
    """The backward's one-wave rows of up to two chunks meet once per row: source gradients on
    sampled rows and dq over every row (the oracle in chunks of rows), T ragged."""
    T, d, r, n, eps = 16384 + 37, 1024, 64, 10, 1e-6
    srcs = synth.values(n, T, d, "bf16", seed=980, scale=(0.5, 4.0), device="cuda")
    q = synth.queries(1, r, 1.0, seed=981, device="cuda")[0].contiguous()
    g = synth.upstream(T, d, seed=982, device="cuda")
    if grad == "bf16":
        g = g.to(torch.bfloat16)
    dsrc = [torch.full((T, d), float("nan"), dtype=g.dtype, device="cuda") for _ in range(n)]
    where = f"lockstep backward d={d} n={n} T={T} grad={grad}"
    say(f"[lockstep] {where}")
    dsrc, dq = lrar.lrar_backward_grad(srcs, q, g, r, eps, dsrc=dsrc)
    torch.cuda.synchronize()
    for i in range(n):
        assert not torch.isnan(dsrc[i].float()).any(), f"{where}: a row of dsrc[{i}] not written"
    rows = sample_rows(T, 24, seed=T)
    s64 = [rows64(s, rows) for s in srcs]
    ds_ref, _ = oracle.backward(s64, f64(q), rows64(g, rows), r, eps)
    for i in range(n):
        if grad == "f32":
            parity.assert_dsrc(rows64(dsrc[i], rows), ds_ref[i], f"{where} dsrc[{i}]")
        else:
            parity.assert_dsrc_bf16(rows64(dsrc[i], rows), ds_ref[i], f"{where} dsrc[{i}]")
    dq_ref = np.zeros(r)
    bound = 0.0
    q64 = f64(q)
    for c0 in range(0, T, 4096):
        sl = slice(c0, c0 + 4096)
        c64 = [f64(s[sl]) for s in srcs]
        g64 = f64(g[sl])
        _, dq_c = oracle.backward(c64, q64, g64, r, eps)
        dq_ref += dq_c
        h_c, a_c = oracle.forward(c64, q64, r, eps)
        bound += parity.dq_bound(c64, q64, g64, a_c, h_c, r, eps)
    parity.assert_dq(f64(dq), dq_ref, bound, where + " dq")
