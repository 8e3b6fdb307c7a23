"""Parity at the full workload sizes, in the launch configuration bench.py times.

The kernels run on every row; the oracle computes sampled rows one by one (first, last, the
ragged end and random rows), and the comparison uses the same element-wise bars as the
small-size tests. The backward's query gradient sums all rows, so the oracle computes it over
every row in chunks of rows (the sum is the definition of dq) and the two sums are compared.
Inputs are drawn on the device from the seeded generators and only the sampled rows are
copied back.
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


def dev_sources(n, T, d, seed, scale):
    return synth.values(n, T, d, "bf16", seed, scale=scale, device="cuda")


def rows64(t, rows):
    idx = torch.as_tensor(rows, device=t.device)
    return f64(t.index_select(0, idx))


def check_read_rows(srcs, q, r, eps, out, alpha, rows, where):
    s64 = [rows64(s, rows) for s in srcs]
    h_ref, a_ref = oracle.forward(s64, f64(q), r, eps)
    parity.assert_weights(rows64(alpha, rows), a_ref, where + " alpha")
    parity.assert_read(rows64(out, rows), h_ref, a_ref, s64, "bf16", where + " h")


@pytest.mark.parametrize("n", [1, 2, 25, 49])
def test_full_routing_d1024(n):
    """The full-routing step's reads: T = 8 x 2048, d = 1024, r = 64."""
    T, d, r, eps = 8 * 2048, 1024, 64, 1e-6
    srcs = dev_sources(n, T, d, seed=500, scale=(0.5, 2.0))
    q = synth.queries(1, r, 1.0, seed=501, device="cuda")[0].contiguous()
    say(f"[full] full routing T={T} d={d} r={r} n={n}")
    out, alpha = lrar.lrar_forward(srcs, q, r, eps, alpha=True)
    torch.cuda.synchronize()
    check_read_rows(srcs, q, r, eps, out, alpha, sample_rows(T, 48, seed=n), f"d1024 n={n}")


@pytest.mark.parametrize("r", [16, 64, 512, 2048])
@pytest.mark.parametrize("variant", ["auto", "two_pass"])
def test_block_routing_d2048(r, variant):
    """Block routing: T = 16 x 4096, d = 2048, the widest site (9 sources) and the capacity
    site (10)."""
    T, d, eps = 16 * 4096, 2048, 1e-6
    srcs = dev_sources(10, T, d, seed=510, scale=(0.5, 4.0))
    q = synth.queries(1, r, 1.0, seed=511 + r, device="cuda")[0].contiguous()
    for n in (9, 10):
        say(f"[full] block routing T={T} d={d} r={r} n={n} {variant}")
        out, alpha = lrar.lrar_forward(srcs[:n], q, r, eps, alpha=True, variant=variant)
        torch.cuda.synchronize()
        check_read_rows(srcs[:n], q, r, eps, out, alpha, sample_rows(T, 32, seed=r + n),
                        f"d2048 r={r} n={n}")


@pytest.mark.parametrize("r", [64, 1792, 7168])
def test_production_width_single_pass(r):
    """Production width: T = 32768, d = 7168, 9 sources."""
    T, d, eps = 32768, 7168, 1e-6
    srcs = dev_sources(9, T, d, seed=520, scale=(0.5, 4.0))
    q = synth.queries(1, r, 1.0, seed=521 + r, device="cuda")[0].contiguous()
    say(f"[full] production width T={T} d={d} r={r} n=9")
    out, alpha = lrar.lrar_forward(srcs, q, r, eps, alpha=True)
    torch.cuda.synchronize()
    check_read_rows(srcs, q, r, eps, out, alpha, sample_rows(T, 24, seed=r), f"d7168 r={r}")


@pytest.mark.parametrize("acc_dtype", [torch.float32, torch.bfloat16])
def test_production_width_two_phase(acc_dtype):
    """The two-phase schedule at production width: Phase 1 batches 12 site queries against 8
    cached block sources (T = 32768, d = 7168, r = 1792); Phase 2 merges each site's partial
    sum. Phase 1's statistics are checked against the oracle's on sampled rows (fp32 acc), and
    every merged site against the oracle's single read over all 9 sources."""
    T, d, r, eps, nq = 32768, 7168, 1792, 1e-6, 12
    srcs = dev_sources(9, T, d, seed=530, scale=(0.5, 4.0))
    qs = synth.queries(nq, r, 1.0, seed=531, device="cuda")
    say(f"[full] phase 1 T={T} d={d} r={r} n_inter=8 nq={nq} acc={acc_dtype}")
    m, l, acc = lrar.lrar_forward_stats(srcs[:8], qs, r, eps, acc_dtype=acc_dtype)
    torch.cuda.synchronize()
    rows = sample_rows(T, 12, seed=532)
    s64 = [rows64(s, rows) for s in srcs]
    q64 = f64(qs)
    if acc_dtype == torch.float32:
        m_o, l_o, acc_o = oracle.stats(s64[:8], q64, r, eps)
        for s in range(nq):
            z_o, _ = oracle.scores(s64[:8], q64[s], r, eps)
            parity.assert_stats(rows64(m[s], rows), rows64(l[s], rows), rows64(acc[s], rows),
                                m_o[s], l_o[s], acc_o[s], z_o, s64[:8], "f32",
                                f"phase 1 query {s}")
    for s in (0, 5, nq - 1):
        say(f"[full] phase 2 site {s}")
        out = lrar.lrar_merge(m[s], l[s], acc[s], srcs[8:9], qs[s].contiguous(), r, eps,
                              io_dtype=torch.bfloat16)
        torch.cuda.synchronize()
        h_ref, a_ref = oracle.forward(s64, q64[s], r, eps)
        y = rows64(out, rows)
        if acc_dtype == torch.float32:
            parity.assert_read(y, h_ref, a_ref, s64, "bf16", f"two-phase site {s}")
        else:
            # a bf16 accumulator adds one bf16 rounding of the Phase-1 partial sum
            mag = sum(a_ref[:, i:i + 1] * np.abs(s64[i]) for i in range(9))
            tol = 2 * parity.ulp_bf16(h_ref) + parity.ulp_bf16(mag) + 12 * parity.U * mag
            parity._report(np.abs(y - h_ref), tol, f"two-phase bf16-acc site {s}")


def test_backward_d4096():
    """Backward of block routing: T = 16384, d = 4096, r = 1024, 10 sources, fp32 gradients.
    Source gradients on sampled rows; dq over all rows."""
    T, d, r, n, eps = 16384, 4096, 1024, 10, 1e-6
    srcs = dev_sources(n, T, d, seed=540, scale=(0.5, 4.0))
    q = synth.queries(1, r, 1.0, seed=541, device="cuda")[0].contiguous()
    g = synth.upstream(T, d, seed=542, device="cuda")
    say(f"[full] backward T={T} d={d} r={r} n={n}")
    dsrc, dq = lrar.lrar_backward(srcs, q, g, r, eps)
    torch.cuda.synchronize()
    rows = sample_rows(T, 16, seed=543)
    s64 = [rows64(s, rows) for s in srcs]
    ds_ref, _ = oracle.backward(s64, f64(q), rows64(g, rows), r, eps)
    for i in range(n):
        parity.assert_dsrc(rows64(dsrc[i], rows), ds_ref[i], f"dsrc[{i}]")
    # dq: the oracle over every row, in chunks, with the tolerance's magnitude sum alongside
    dq_ref = np.zeros(r)
    bound = 0.0
    q64 = f64(q)
    for c0 in range(0, T, 2048):
        sl = slice(c0, c0 + 2048)
        c64 = [f64(s[sl]) for s in srcs]
        g64 = f64(g[sl])
        _, dq_c = oracle.backward(c64, q64, g64, r, eps)
        dq_ref += dq_c
        h_c, a_c = oracle.forward(c64, q64, r, eps)
        bound += parity.dq_bound(c64, q64, g64, a_c, h_c, r, eps)
    parity.assert_dq(f64(dq), dq_ref, bound)
