"""lrar_forward_stats (Phase 1) and lrar_merge (Phase 2) on the GPU against the oracle."""
import numpy as np
import pytest
import torch

import oracle
import parity
import transformer_depth_wise_lrar_amd as lrar
from gpu_util import f64, io_of, needs_gpu, query, say, sources

pytestmark = [pytest.mark.gpu, needs_gpu]


def check_stats(srcs, qs, r, eps, acc_dtype, where):
    qs = qs.reshape(-1, r) if qs.dim() == 1 else qs
    say(f"[stats] {where} T={srcs[0].shape[0]} d={srcs[0].shape[1]} r={r} n={len(srcs)} "
        f"nq={qs.shape[0]} acc={acc_dtype}")
    m, l, acc = lrar.lrar_forward_stats(srcs, qs, r, eps, acc_dtype=acc_dtype)
    torch.cuda.synchronize()
    s64 = [f64(s) for s in srcs]
    q64 = f64(qs)
    m_o, l_o, acc_o = oracle.stats(s64, q64, r, eps)
    m_g, l_g, acc_g = f64(m), f64(l), f64(acc)
    for s in range(qs.shape[0]):
        z_o, _ = oracle.scores(s64, q64[s], r, eps)
        parity.assert_stats(m_g[s], l_g[s], acc_g[s], m_o[s], l_o[s], acc_o[s], z_o, s64,
                            "bf16" if acc_dtype == torch.bfloat16 else "f32",
                            f"{where} query {s}")
    return m, l, acc


@pytest.mark.parametrize("nq", [1, 2, 3, 8, 12, 16, 20])
@pytest.mark.parametrize("acc_dtype", [torch.float32, torch.bfloat16])
def test_stats_against_oracle(nq, acc_dtype):
    srcs = sources(5, 45, 1024, "bf16", seed=100, scale=(0.5, 4.0))
    qs = query(64, seed=101, nq=nq)
    check_stats(srcs, qs, 64, 1e-6, acc_dtype, f"nq={nq}")


@pytest.mark.parametrize("d,r", [(513, 100), (2048, 512), (7168, 1792), (64, 16)])
@pytest.mark.parametrize("io", ["bf16", "f32"])
def test_stats_shapes(d, r, io):
    srcs = sources(4, 23, d, io, seed=102, scale=(0.5, 4.0))
    qs = query(r, seed=103, nq=3)
    check_stats(srcs, qs, r, 1e-6, torch.float32, f"d{d} r{r}")


@pytest.mark.parametrize("n", [3, 8])
@pytest.mark.parametrize("io", ["bf16", "f32"])
@pytest.mark.parametrize("acc_dtype", [torch.float32, torch.bfloat16])
def test_stats_full_group_ragged_width(n, io, acc_dtype):
    """A full group of 12 queries (the kernel variant with no query-count branches) on a width
    that ends in a partial chunk: the lanes past the row's end load and store the row's last
    unit, which must leave every element equal to the oracle's."""
    srcs = sources(n, 37, 1000, io, seed=106, scale=(0.5, 4.0))
    qs = query(200, seed=107, nq=12)
    check_stats(srcs, qs, 200, 1e-6, acc_dtype, f"full group n={n} d=1000")


def test_stats_strided_queries():
    r = 64
    srcs = sources(3, 31, 1024, "bf16", seed=104)
    Q = torch.randn((4, r + 9), generator=torch.Generator().manual_seed(105)).cuda()
    check_stats(srcs, Q[:, :r], r, 1e-6, torch.float32, "strided queries")


def _merge_case(n_inter, n_extra, d, r, io, acc_dtype, seed):
    """Oracle statistics (rounded to the storage types) merged by the kernel and by the
    oracle; the inputs to both sides are the same float32/bf16 values."""
    T = 41
    inter = sources(n_inter, T, d, io, seed=seed, scale=(0.5, 4.0))
    extra = sources(n_extra, T, d, io, seed=seed + 1, scale=(0.5, 4.0)) if n_extra else []
    q = query(r, seed=seed + 2)
    s64 = [f64(s) for s in inter]
    m_o, l_o, acc_o = oracle.stats(s64, f64(q)[None, :], r, 1e-6)
    m = torch.tensor(m_o[0], dtype=torch.float32, device="cuda")
    l = torch.tensor(l_o[0], dtype=torch.float32, device="cuda")
    acc = torch.tensor(acc_o[0], dtype=torch.float32).to(acc_dtype).cuda()
    say(f"[merge] n_inter={n_inter} n_extra={n_extra} d={d} r={r} io={io} acc={acc_dtype}")
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
                        "merge h")
    # m' is the float32 rounding of the exact maximum; l' is relative to that m'
    m2g = f64(m2)
    assert np.all(np.abs(m2g - m_ref) <= 2.0 ** -23 * np.abs(m_ref) + 1e-12)
    l_resc = l_ref * np.exp(m_ref - m2g)
    assert np.all(np.abs(f64(l2) - l_resc) <= 4 * parity.U * l_resc)


@pytest.mark.parametrize("n_inter,n_extra", [(1, 1), (8, 1), (3, 0), (2, 4)])
@pytest.mark.parametrize("io", ["bf16", "f32"])
@pytest.mark.parametrize("acc_dtype", [torch.float32, torch.bfloat16])
def test_merge_against_oracle(n_inter, n_extra, io, acc_dtype):
    _merge_case(n_inter, n_extra, 1024, 64, io, acc_dtype, seed=110 + n_inter)


@pytest.mark.parametrize("d,r", [(513, 64), (7168, 7168), (2048, 16), (2048, 509)])
def test_merge_shapes(d, r):
    _merge_case(4, 1, d, r, "bf16", torch.float32, seed=120)


@pytest.mark.parametrize("split", [1, 4, 8])
def test_two_phase_equals_single_pass(split):
    """Phase 1 over the first `split` sources for a batch of site queries, then Phase 2 with
    the rest, against the oracle's single read over all sources (the two-phase property)."""
    d, r, T = 2048, 512, 57
    srcs = sources(9, T, d, "bf16", seed=130, scale=(0.5, 4.0))
    qs = query(r, seed=131, nq=6)
    m, l, acc = lrar.lrar_forward_stats(srcs[:split], qs, r, 1e-6)
    s64 = [f64(s) for s in srcs]
    for s in range(6):
        say(f"[two-phase] split={split} site={s}")
        out = lrar.lrar_merge(m[s], l[s], acc[s], srcs[split:], qs[s].contiguous(), r, 1e-6,
                              io_dtype=torch.bfloat16)
        torch.cuda.synchronize()
        h_ref, a_ref = oracle.forward(s64, f64(qs[s]), r, 1e-6)
        # the stored statistics add one float32 rounding of acc (and of l) to the read
        parity.assert_read(f64(out), h_ref, a_ref, s64, "bf16", f"two-phase site {s}")
