"""Reads of many rows: the one-pass spread-key reads, and the one-pass reads whose key comes
from the row units of one wave, are cut into several launches over consecutive row ranges (at
most a fixed number of tiles per row group each); other reads and merges run as one launch over
the same rows.

These tests fill the outputs with NaN first and then check that every row was written, that
every row's weights sum to 1, and that rows on both sides of the launch boundaries (and the
ragged last row) match the oracle.
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


def boundary_rows(T, parts=12):
    """Rows around every 1/parts of T, the ends, and random rows (sorted, distinct)."""
    rows = set(sample_rows(T, 16, seed=T))
    for k in range(1, parts):
        c = T * k // parts
        rows.update(x for x in range(c - 2, c + 2) if 0 <= x < T)
    rows.update((0, 1, T - 2, T - 1))
    return sorted(rows)


def rows64(t, rows):
    idx = torch.as_tensor(rows, device=t.device)
    return f64(t.index_select(0, idx))


@pytest.mark.parametrize("d,r,n,T", [
    (2048, 64, 9, 65536 + 37),     # cut: one wave per row, short spread key, drained one ahead
    (2048, 64, 1, 65536 + 37),     # cut: one source, the two-stage tile alternation
    (7168, 64, 3, 32768 + 5),      # cut: four waves per row, two-deep ring
    (7168, 64, 9, 32768 + 5),      # cut: four waves per row, drained one ahead
    (2048, 512, 3, 65536 + 37),    # cut: 16-element key pieces, one source ahead
    (2048, 2048, 3, 65536 + 37),   # cut: key from the row units of one wave
    (7168, 1792, 3, 32768 + 5),    # one launch: the row's two waves exchange key sums
])
def test_every_row_written(d, r, n, T):
    eps = 1e-6
    srcs = synth.values(n, T, d, "bf16", seed=900 + n, scale=(0.5, 4.0), device="cuda")
    q = synth.queries(1, r, 1.0, seed=901 + r, device="cuda")[0].contiguous()
    out = torch.full((T, d), float("nan"), dtype=torch.bfloat16, device="cuda")
    alpha = torch.full((T, n), float("nan"), dtype=torch.float32, device="cuda")
    say(f"[launches] read T={T} d={d} r={r} n={n}")
    lrar.lrar_forward(srcs, q, r, eps, out=out, alpha=alpha)
    torch.cuda.synchronize()
    assert not bool(torch.isnan(out).any()), "rows left unwritten"
    sums = alpha.double().sum(dim=1)
    assert float((sums - 1.0).abs().max()) <= 1e-6 * n, "weights of some rows do not sum to 1"
    rows = boundary_rows(T)
    s64 = [rows64(s, rows) for s in srcs]
    h_ref, a_ref = oracle.forward(s64, f64(q), r, eps)
    where = f"T={T} d={d} r={r} n={n}"
    parity.assert_weights(rows64(alpha, rows), a_ref, where + " alpha")
    parity.assert_read(rows64(out, rows), h_ref, a_ref, s64, "bf16", where + " h")


def test_merge_every_row_written():
    """Phase 2 over many rows: the merge of (m, l, acc) with one extra source."""
    T, d, r, eps = 65536 + 37, 2048, 512, 1e-6
    srcs = synth.values(4, T, d, "bf16", seed=950, scale=(0.5, 4.0), device="cuda")
    q = synth.queries(1, r, 1.0, seed=951, device="cuda")[0].contiguous()
    say(f"[launches] merge T={T} d={d} r={r}")
    m, l, acc = lrar.lrar_forward_stats(srcs[:3], q[None, :].contiguous(), r, eps)
    out = torch.full((T, d), float("nan"), dtype=torch.bfloat16, device="cuda")
    lrar.lrar_merge(m[0], l[0], acc[0], srcs[3:], q, r, eps, out=out)
    torch.cuda.synchronize()
    assert not bool(torch.isnan(out).any()), "rows left unwritten"
    rows = boundary_rows(T)
    s64 = [rows64(s, rows) for s in srcs]
    h_ref, a_ref = oracle.forward(s64, f64(q), r, eps)
    parity.assert_read(rows64(out, rows), h_ref, a_ref, s64, "bf16", f"merge T={T}")


@pytest.mark.parametrize("d,r,n,T", [(2048, 64, 9, 65536 + 37), (7168, 64, 3, 32768 + 5),
                                     (2048, 2048, 3, 65536 + 37)])
def test_cut_read_matches_uncut_slices(d, r, n, T):
    """Each row's result depends on that row alone: rows of a read cut into several launches
    are bitwise equal to the same rows read on their own (a slice short enough for one
    launch), at the launch boundaries and at the ragged end."""
    eps = 1e-6
    srcs = synth.values(n, T, d, "bf16", seed=970 + n, scale=(0.5, 4.0), device="cuda")
    q = synth.queries(1, r, 1.0, seed=971, device="cuda")[0].contiguous()
    say(f"[launches] cut vs uncut T={T} d={d} r={r} n={n}")
    out, alpha = lrar.lrar_forward(srcs, q, r, eps, alpha=True)
    for a in (0, T // 4 - 3, T // 2 - 5, T - 700):
        b = min(T, a + 640)
        o2, a2 = lrar.lrar_forward([s[a:b] for s in srcs], q, r, eps, alpha=True)
        torch.cuda.synchronize()
        assert torch.equal(out[a:b], o2), f"rows {a}..{b - 1}: h differs from the uncut read"
        assert torch.equal(alpha[a:b], a2), f"rows {a}..{b - 1}: weights differ"
