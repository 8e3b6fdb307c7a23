"""lrar_backward_grad with bf16 gradients (dout and dsrc bf16, dq float32) on the GPU against
the oracle. The oracle takes the bf16 upstream gradient decoded exactly; the source gradients
are held to the float32 bar plus one bf16 ulp (one rounding of the float32 result)."""
import numpy as np
import pytest
import torch

import oracle
import parity
import transformer_depth_wise_lrar_amd as lrar
from gpu_util import f64, needs_gpu, query, sample_rows, say, sources
from transformer_depth_wise_lrar_amd import synth

pytestmark = [pytest.mark.gpu, needs_gpu]


def check(srcs, q, r, eps, accumulate, where, seed=0):
    T, d = srcs[0].shape
    say(f"[backward bf16] {where} T={T} d={d} r={r} n={len(srcs)} accumulate={accumulate}")
    dout = synth.upstream(T, d, seed, device="cpu").to(torch.bfloat16).cuda()
    prior = None
    dsrc = None
    if accumulate:
        prior = [torch.randn((T, d), generator=torch.Generator().manual_seed(seed + i))
                 .to(torch.bfloat16).cuda() for i in range(len(srcs))]
        dsrc = [p.clone() for p in prior]
    dsrc, dq = lrar.lrar_backward_grad(srcs, q, dout, r, eps, dsrc=dsrc, accumulate=accumulate)
    torch.cuda.synchronize()
    assert all(g.dtype == torch.bfloat16 for g in dsrc)
    s64 = [f64(s) for s in srcs]
    g64 = f64(dout)
    ds_ref, dq_ref = oracle.backward(s64, f64(q), g64, r, eps)
    for i in range(len(srcs)):
        ref = ds_ref[i] + (f64(prior[i]) if accumulate else 0.0)
        parity.assert_dsrc_bf16(f64(dsrc[i]), ref, f"{where} dsrc[{i}]")
    h, al = oracle.forward(s64, f64(q), r, eps)
    parity.assert_dq(f64(dq), dq_ref, parity.dq_bound(s64, f64(q), g64, al, h, r, eps),
                     f"{where} dq")


@pytest.mark.parametrize("io", ["bf16", "f32"])
@pytest.mark.parametrize("d,r", [(64, 16), (1024, 64), (513, 100), (4096, 1024), (7168, 1792),
                                 (16384, 64)])
@pytest.mark.parametrize("accumulate", [False, True])
def test_backward_bf16_grads(io, d, r, accumulate):
    """Every tile shape and the element path (d = 513), bf16 and float32 sources (float32 rows
    of 16384 run the one-wave-per-row backward), with and without accumulation into existing
    bf16 gradients."""
    srcs = sources(5, 29, d, io, seed=800 + d, scale=(0.5, 4.0))
    check(srcs, query(r, seed=801), r, 1e-6, accumulate, f"{io} d{d} r{r}", seed=802)


def test_backward_bf16_f32_entry_points_agree():
    """lrar_backward_grad with float32 gradients is lrar_backward, bit for bit."""
    srcs = sources(6, 40, 1024, "bf16", seed=810)
    q = query(64, seed=811)
    dout = synth.upstream(40, 1024, 812, device="cpu").cuda()
    say("[backward bf16] f32 entry points agree")
    a, dqa = lrar.lrar_backward(srcs, q, dout, 64, 1e-6)
    b, dqb = lrar.lrar_backward_grad(srcs, q, dout, 64, 1e-6)
    torch.cuda.synchronize()
    assert torch.equal(dqa, dqb) and all(torch.equal(x, y) for x, y in zip(a, b))


def test_backward_bf16_full_size_d4096():
    """T = 16384, d = 4096, r = 1024, 10 sources, bf16 gradients: source gradients on sampled
    rows, dq over all rows (the oracle in chunks of rows)."""
    T, d, r, n, eps = 16384, 4096, 1024, 10, 1e-6
    srcs = synth.values(n, T, d, "bf16", 820, scale=(0.5, 4.0), device="cuda")
    q = synth.queries(1, r, 1.0, seed=821, device="cuda")[0].contiguous()
    g = synth.upstream(T, d, seed=822, device="cuda").to(torch.bfloat16)
    say(f"[backward bf16] full size T={T} d={d} r={r} n={n}")
    dsrc, dq = lrar.lrar_backward_grad(srcs, q, g, r, eps)
    torch.cuda.synchronize()
    rows = sample_rows(T, 16, seed=823)
    idx = torch.as_tensor(rows, device="cuda")
    pick = lambda t: f64(t.index_select(0, idx))  # noqa: E731
    s64 = [pick(s) for s in srcs]
    ds_ref, _ = oracle.backward(s64, f64(q), pick(g), r, eps)
    for i in range(n):
        parity.assert_dsrc_bf16(pick(dsrc[i]), ds_ref[i], f"dsrc[{i}]")
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
