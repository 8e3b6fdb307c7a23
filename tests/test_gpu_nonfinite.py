"""Non-finite source values go through the read as they go through the oracle's arithmetic
(LR-AttnRes paper §3.1 routing equation, §3.3 routing keys; the oracle is the plain fp64
definition): a NaN or an infinity in a value column reaches only that column of h (an
infinity from the source with the row's largest weight stays an infinity of the same sign,
+inf and -inf from two sources give NaN), and the row's weights are unchanged; a NaN or an
infinity in a key column makes that source's score NaN, so the row's weights and every
column of its h are NaN. Rows without such values match the oracle as usual.

Every kernel shape of the forward read is taken: one-wave rows (d = 1024, 2048), rows shared
by four waves with a spread key (d = 7168, r = 64) and by two waves with the key in the row
units (d = 7168, r = 1792), in the online and the two-pass variant, bf16 and fp32.
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
