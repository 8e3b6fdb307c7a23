"""Non-finite source values go through the read as they go through the oracle's arithmetic
(LR-AttnRes paper §3.1 routing equation, §3.3 routing keys; the oracle is the plain fp64
definition): a NaN or an infinity in a value column reaches only that column of h (an
infinity from the source with the row's largest weight stays an infinity of the same sign,
+inf and -inf from two sources give NaN), and the row's weights are unchanged; a NaN or an
infinity in a key column makes that source's score NaN, so the row's weights and every
column of its h are NaN. Rows without such values match the oracle as usual.

Every kernel shape of the forward read is taken: one-wave rows (d = 1024, 2048), rows shared
by four waves with a spread key (d = 7168, r = 64) and by two waves with the key in the row
units (d = 7168, r = 1792), in the online and the two-pass variant, bf16 and fp32. Phase 1 and
the Phase-2 merge take non-finite value columns the same way.
"""
import numpy as np
import pytest
import torch

import oracle
import parity
import transformer_depth_wise_lrar_amd as lrar
from gpu_util import f64, needs_gpu, query, say, sources

pytestmark = [pytest.mark.gpu, needs_gpu]

T = 300
NAN_VAL, INF_VAL, PAIR_VAL, NAN_KEY, INF_KEY = 5, 17, 123, 40, 77


def plant(srcs, q, r, eps):
    """Writes the non-finite values into the device sources; returns the rows they touch."""
    s64 = [f64(s) for s in srcs]
    _, a = oracle.forward(s64, f64(q), r, eps)
    n, d = len(srcs), srcs[0].shape[1]
    order = np.argsort(-a, axis=1)
    c0 = d - r
    col_v = min(3, c0 - 1) if c0 > 0 else None   # a value column outside the key
    with torch.no_grad():
        if col_v is not None:
            srcs[min(1, n - 1)][NAN_VAL, col_v] = float("nan")
            srcs[int(order[INF_VAL, 0])][INF_VAL, col_v] = float("inf")
            if n >= 2:
                srcs[int(order[PAIR_VAL, 0])][PAIR_VAL, col_v] = float("inf")
                srcs[int(order[PAIR_VAL, 1])][PAIR_VAL, col_v] = float("-inf")
        srcs[0][NAN_KEY, d - 1] = float("nan")
        srcs[n - 1][INF_KEY, c0] = float("inf")
    return col_v


def check(out, alpha, srcs, q, r, eps, io, where):
    s64 = [f64(s) for s in srcs]
    h_ref, a_ref = oracle.forward(s64, f64(q), r, eps)
    y = f64(out)
    a = f64(alpha)
    for name, test in (("NaN", np.isnan), ("+inf", np.isposinf), ("-inf", np.isneginf)):
        got, ref = test(y), test(h_ref)
        assert np.array_equal(got, ref), (
            f"{where}: {name} at {np.argwhere(got != ref)[:4].tolist()} (row, column) differs")
    key_rows = [NAN_KEY, INF_KEY]
    assert np.isnan(a[key_rows]).all() and np.isnan(a_ref[key_rows]).all(), where + " key rows"
    rest = np.setdiff1d(np.arange(T), key_rows)
    parity.assert_weights(a[rest], a_ref[rest], where + " alpha")
    finite = np.isfinite(h_ref[rest])
    y_f = np.where(finite, y[rest], 0.0)
    h_f = np.where(finite, h_ref[rest], 0.0)
    s_f = [np.where(np.isfinite(s[rest]), s[rest], 0.0) for s in s64]
    parity.assert_read(y_f, h_f, a_ref[rest], s_f, io, where + " h")


@pytest.mark.parametrize("variant", ["online", "two_pass"])
@pytest.mark.parametrize("d,r,n,io", [(1024, 64, 9, "bf16"), (2048, 512, 10, "bf16"),
                                      (7168, 64, 9, "bf16"), (7168, 1792, 9, "bf16"),
                                      (1024, 64, 5, "f32"), (2048, 2048, 3, "bf16")])
def test_nonfinite_values_and_keys(d, r, n, io, variant):
    eps = 1e-6
    where = f"nonfinite d={d} r={r} n={n} {io} {variant}"
    say(f"[nonfinite] {where}")
    srcs = sources(n, T, d, io, seed=990 + d + n)
    q = query(r, seed=991 + r, std=0.25)
    plant(srcs, q, r, eps)
    dt = srcs[0].dtype
    out = torch.full((T, d), 7.0, dtype=dt, device="cuda")
    alpha = torch.full((T, n), 7.0, dtype=torch.float32, device="cuda")
    lrar.lrar_forward(srcs, q, r, eps, out=out, alpha=alpha, variant=variant)
    torch.cuda.synchronize()
    check(out, alpha, srcs, q, r, eps, io, where)


def same_nonfinite(y, ref, where):
    for name, test in (("NaN", np.isnan), ("+inf", np.isposinf), ("-inf", np.isneginf)):
        got, want = test(y), test(ref)
        assert np.array_equal(got, want), (
            f"{where}: {name} at {np.argwhere(got != want)[:4].tolist()} differs")


def finite_part(*arrays):
    return [np.where(np.isfinite(a), a, 0.0) for a in arrays]


@pytest.mark.parametrize("nq", [3, 12])
@pytest.mark.parametrize("acc_dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("d,r", [(1024, 64), (7168, 1792)])
def test_stats_nonfinite_values(d, r, acc_dtype, nq):
    """Phase 1 (the technical-report summary, "Method"): a NaN in a value column of one source
    makes that column of every query's accumulator NaN, an infinity makes it an infinity of
    the same sign; m and l are untouched."""
    Tq, n, eps = 40, 8, 1e-6
    where = f"stats nonfinite d={d} r={r} acc={acc_dtype} nq={nq}"
    say(f"[nonfinite] {where}")
    srcs = sources(n, Tq, d, "bf16", seed=995 + d)
    qs = query(r, seed=996 + r, std=0.1, nq=nq)
    with torch.no_grad():
        srcs[1][5, 3] = float("nan")
        srcs[2][17, 3] = float("inf")
        srcs[3][23, 4] = float("-inf")
    m, l, acc = lrar.lrar_forward_stats(srcs, qs, r, eps, acc_dtype=acc_dtype)
    torch.cuda.synchronize()
    s64 = [f64(s) for s in srcs]
    q64 = f64(qs)
    m_o, l_o, acc_o = oracle.stats(s64, q64, r, eps)
    m_g, l_g, acc_g = f64(m), f64(l), f64(acc)
    io = "bf16" if acc_dtype == torch.bfloat16 else "f32"
    for s in range(nq):
        same_nonfinite(acc_g[s], acc_o[s], f"{where} query {s} acc")
        assert np.isnan(acc_o[s][5, 3]) and np.isposinf(acc_o[s][17, 3])
        z_o, _ = oracle.scores(s64, q64[s], r, eps)
        a_g, a_o = finite_part(acc_g[s], acc_o[s])
        parity.assert_stats(m_g[s], l_g[s], a_g, m_o[s], l_o[s], a_o, z_o, finite_part(*s64),
                            io, f"{where} query {s}")


@pytest.mark.parametrize("acc_dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("d,r", [(1024, 64), (7168, 1792)])
def test_merge_nonfinite_values(d, r, acc_dtype):
    """Phase 2: a NaN in the prior accumulator or an infinity in the partial sum's value
    columns reaches only that column of h."""
    Tm, eps = 41, 1e-6
    where = f"merge nonfinite d={d} r={r} acc={acc_dtype}"
    say(f"[nonfinite] {where}")
    inter = sources(4, Tm, d, "bf16", seed=997)
    extra = sources(1, Tm, d, "bf16", seed=998)
    q = query(r, seed=999, std=0.1)
    s64 = [f64(s) for s in inter]
    m_o, l_o, acc_o = oracle.stats(s64, f64(q)[None, :], r, eps)
    acc_o = acc_o[0].copy()
    acc_o[5, 3] = np.nan
    m = torch.tensor(m_o[0], dtype=torch.float32, device="cuda")
    l = torch.tensor(l_o[0], dtype=torch.float32, device="cuda")
    acc = torch.tensor(acc_o, dtype=torch.float32).to(acc_dtype).cuda()
    with torch.no_grad():
        extra[0][17, 3] = float("inf")
    out = lrar.lrar_merge(m, l, acc, extra, q, r, eps, io_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    e64 = [f64(s) for s in extra]
    m_in, l_in, acc_in = f64(m), f64(l), f64(acc)
    h_ref, m_ref, l_ref = oracle.merge(m_in, l_in, acc_in, e64, f64(q), r, eps)
    y = f64(out)
    same_nonfinite(y, h_ref, where)
    assert np.isnan(h_ref[5, 3]) and np.isposinf(h_ref[17, 3])
    z_e, _ = oracle.scores(e64, f64(q), r, eps)
    w_extra = np.exp(z_e - m_ref[:, None]) / l_ref[:, None]
    w_prior = l_in * np.exp(m_in - m_ref) / l_ref
    y_f, h_f, an_f = finite_part(y, h_ref, acc_in / l_in[:, None])
    parity.assert_merge(y_f, h_f, w_prior, an_f, w_extra, finite_part(*e64), "bf16", where)
