"""lrar_backward on the GPU against the oracle."""
import numpy as np
import pytest
import torch

import oracle
import parity
import transformer_depth_wise_lrar_amd as lrar
from gpu_util import f64, needs_gpu, query, say, sources
from transformer_depth_wise_lrar_amd import synth

pytestmark = [pytest.mark.gpu, needs_gpu]


def check_backward(srcs, q, r, eps, accumulate, where, seed=0):
    T, d = srcs[0].shape
    say(f"[backward] {where} T={T} d={d} r={r} n={len(srcs)} accumulate={accumulate}")
    dout = synth.upstream(T, d, seed, device="cpu").cuda()
    prior = None
    dsrc = None
    if accumulate:
        prior = [torch.randn((T, d), generator=torch.Generator().manual_seed(seed + i)).cuda()
                 for i in range(len(srcs))]
        dsrc = [p.clone() for p in prior]
    dsrc, dq = lrar.lrar_backward(srcs, q, dout, r, eps, dsrc=dsrc, accumulate=accumulate)
    torch.cuda.synchronize()
    s64 = [f64(s) for s in srcs]
    g64 = f64(dout)
    ds_ref, dq_ref = oracle.backward(s64, f64(q), g64, r, eps)
    for i in range(len(srcs)):
        ref = ds_ref[i] + (f64(prior[i]) if accumulate else 0.0)
        parity.assert_dsrc(f64(dsrc[i]), ref, f"{where} dsrc[{i}]")
    h, al = oracle.forward(s64, f64(q), r, eps)
    parity.assert_dq(f64(dq), dq_ref, parity.dq_bound(s64, f64(q), g64, al, h, r, eps),
                     f"{where} dq")
    return dsrc, dq


@pytest.mark.parametrize("d,r", [(1024, 64), (4096, 1024), (2048, 2048), (513, 100),
                                 (64, 16), (7168, 1792)])
@pytest.mark.parametrize("n", [1, 2, 10])
def test_backward_shapes(d, r, n):
    srcs = sources(n, 33, d, "bf16", seed=200 + n, scale=(0.5, 4.0))
    check_backward(srcs, query(r, seed=201), r, 1e-6, False, f"d{d} r{r}", seed=202)


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_backward_accumulate(io):
    srcs = sources(4, 70, 1024, io, seed=210)
    check_backward(srcs, query(64, seed=211), 64, 1e-6, True, "accumulate", seed=212)


def test_backward_full_routing_49_sources():
    srcs = sources(49, 21, 1024, "bf16", seed=220)
    check_backward(srcs, query(64, seed=221), 64, 1e-6, False, "n=49", seed=222)


def test_backward_strided_and_repeated():
    base = sources(2, 29, 1024, "bf16", seed=230)
    wide = sources(1, 29, 1024, "bf16", seed=231, row_stride=1024 + 8)
    check_backward([base[0], wide[0], base[0], base[1]], query(64, seed=232), 64, 1e-6, False,
                   "strided+repeated", seed=233)


def test_backward_deterministic():
    srcs = sources(10, 300, 4096, "bf16", seed=240, scale=(0.5, 4.0))
    q = query(1024, seed=241)
    dout = synth.upstream(300, 4096, 242, device="cpu").cuda()
    a, dqa = lrar.lrar_backward(srcs, q, dout, 1024, 1e-6)
    b, dqb = lrar.lrar_backward(srcs, q, dout, 1024, 1e-6)
    torch.cuda.synchronize()
    assert torch.equal(dqa, dqb)
    assert all(torch.equal(x, y) for x, y in zip(a, b))


@pytest.mark.parametrize("d,r,io", [(4096, 512, "f32"), (12288, 256, "bf16"),
                                    (16384, 16384, "bf16"), (8192, 4000, "f32")])
def test_backward_wide_rows(d, r, io):
    """Rows shared by the four waves of a workgroup, up to the widest tile (32 chunks)."""
    srcs = sources(3, 19, d, io, seed=250, scale=(0.5, 4.0))
    check_backward(srcs, query(r, seed=251), r, 1e-6, False, f"wide d{d} r{r} {io}", seed=252)


@pytest.mark.parametrize("d,io", [(4096, "bf16"), (8192, "f32"), (8200, "f32"), (16392, "bf16")])
@pytest.mark.parametrize("r", [1, 2, 16])
def test_backward_key_term_cancellation(d, r, io):
    """Small keys parallel to the query: d z / d k_j = (q_j - (z / r) kbar_j) / rho is then
    q_j eps / (|k|^2 / r + eps) / rho, a small difference of two large terms (LR-AttnRes paper,
    App. B.3, Lemma 2; at r = 1 every key is parallel to q). With |k| / sqrt(r) in [0.01, 0.05]
    and eps = 1e-6 the terms are 400-25000 times their difference, which float32 coefficients
    of the two terms (one rounding each) do not resolve to the 1e-5 bar. Row tiles (up to 8192
    fp32 / 16384 bf16 columns) and the one-wave-per-row path past them."""
    T, n = 40, 4
    qt = synth.queries(1, r, 1.0, 261, device="cpu")[0]
    srcs = []
    for i, s in enumerate(synth.values(n, T, d, io, 260 + d + r, scale=(0.5, 4.0), device="cpu")):
        g = torch.Generator().manual_seed(270 + i)
        mag = 0.01 + 0.04 * torch.rand((T, 1), generator=g)
        sign = torch.where(torch.rand((T, 1), generator=g) < 0.5, -1.0, 1.0)
        s[:, d - r:] = (mag * sign * (r ** 0.5) * qt / qt.norm()).to(s.dtype)
        srcs.append(s.cuda())
    check_backward(srcs, qt.cuda(), r, 1e-6, False, f"parallel small keys d{d} r{r} {io}",
                   seed=262)
