"""The forward's saved statistics (lrar_forward_save: per row the scores z_i and 1 / rho_i) and
the backward that reuses them (lrar_backward_saved) on the GPU against the oracle (LR-AttnRes
paper App. I, "Implementation": the kernel keeps normalization and softmax statistics for its
backward; App. B.3 for the gradients)."""
import numpy as np
import pytest
import torch

import oracle
import parity
import transformer_depth_wise_lrar_amd as lrar
from gpu_util import f64, io_of, needs_gpu, query, say, sources
from transformer_depth_wise_lrar_amd import synth

pytestmark = [pytest.mark.gpu, needs_gpu]

# (d, r, io, source row stride or None): every path of the read and of the backward
SHAPES = [
    (1024, 64, "bf16", None),     # spread key, two rows per tile
    (2048, 512, "bf16", None),    # key units in the last slot
    (2048, 2048, "bf16", None),   # r = d (standard AttnRes), one source in flight
    (4096, 1024, "bf16", None),   # rows shared by four waves, key stash in the backward
    (7168, 1792, "bf16", None),   # production width
    (1024, 100, "f32", None),
    (513, 200, "bf16", None),     # element path (unaligned width)
    (2560, 640, "bf16", 2561),    # element path past a tile (odd stride)
    (16392, 64, "bf16", None),    # vector rows past the widest tile
]
IDS = [f"d{d}-r{r}-{io}-ld{ld}" for d, r, io, ld in SHAPES]


def check_saved(saved, srcs, q, r, eps, where):
    z_o, rho_o = oracle.scores([f64(s) for s in srcs], f64(q), r, eps)
    n = len(srcs)
    sv = f64(saved)
    z, rinv = sv[:, :n], sv[:, n:2 * n]
    # float64 scores in another summation order: a few ulp of the sum of |q_j k_j| / rho
    assert np.all(np.abs(z - z_o) <= 1e-12 * np.maximum(1.0, np.abs(z_o)) + 1e-12), where + " z"
    assert np.all(np.abs(rinv * rho_o - 1.0) <= 1e-13), where + " 1/rho"


@pytest.mark.parametrize("d,r,io,ld", SHAPES, ids=IDS)
@pytest.mark.parametrize("variant", ["auto", "two_pass"])
def test_forward_save(d, r, io, ld, variant):
    """The saved z_i and 1 / rho_i equal the oracle's; h is bit for bit lrar_forward's."""
    n = 5
    srcs = sources(n, 19, d, io, seed=1800 + d, scale=(0.5, 4.0), row_stride=ld)
    q = query(r, seed=1801)
    say(f"[forward_save] d={d} r={r} io={io} ld={ld} variant={variant}")
    out, saved = lrar.lrar_forward_save(srcs, q, r, 1e-6, variant=variant)
    ref, _ = lrar.lrar_forward(srcs, q, r, 1e-6, variant=variant)
    torch.cuda.synchronize()
    assert torch.equal(out, ref)
    check_saved(saved, srcs, q, r, 1e-6, f"d{d} r{r}")


@pytest.mark.parametrize("n", [1, 3, 13, 49])
def test_forward_save_source_counts(n):
    """Every ring of the headline read (one source, two-deep, three-deep)."""
    srcs = sources(n, 37, 1024, "bf16", seed=1810 + n)
    q = query(64, seed=1811)
    say(f"[forward_save] n={n}")
    out, saved = lrar.lrar_forward_save(srcs, q, 64, 1e-6)
    torch.cuda.synchronize()
    check_saved(saved, srcs, q, 64, 1e-6, f"n={n}")
    s64 = [f64(s) for s in srcs]
    h_ref, a_ref = oracle.forward(s64, f64(q), 64, 1e-6)
    parity.assert_read(f64(out), h_ref, a_ref, s64, "bf16", f"n={n} h")


@pytest.mark.parametrize("d,r,io,ld", SHAPES, ids=IDS)
@pytest.mark.parametrize("grad", ["f32", "bf16"])
@pytest.mark.parametrize("accumulate", [False, True])
def test_backward_saved(d, r, io, ld, grad, accumulate):
    """lrar_backward_saved from lrar_forward_save's statistics against the oracle's backward,
    with the bars of lrar_backward (plus one bf16 ulp for bf16 gradients)."""
    T, n, eps = 21, 6, 1e-6
    srcs = sources(n, T, d, io, seed=1900 + d, scale=(0.5, 4.0), row_stride=ld)
    q = query(r, seed=1901)
    gdt = torch.float32 if grad == "f32" else torch.bfloat16
    dout = synth.upstream(T, d, 1902, device="cpu").to(gdt).cuda()
    prior = dsrc = None
    if accumulate:
        prior = [torch.randn((T, d), generator=torch.Generator().manual_seed(1903 + i))
                 .to(gdt).cuda() for i in range(n)]
        dsrc = [p.clone() for p in prior]
    say(f"[backward_saved] d={d} r={r} io={io} ld={ld} grad={grad} accumulate={accumulate}")
    _, saved = lrar.lrar_forward_save(srcs, q, r, eps)
    dsrc, dq = lrar.lrar_backward_saved(srcs, q, saved, dout, r, dsrc=dsrc,
                                        accumulate=accumulate)
    torch.cuda.synchronize()
    s64 = [f64(s) for s in srcs]
    g64 = f64(dout)
    ds_ref, dq_ref = oracle.backward(s64, f64(q), g64, r, eps)
    for i in range(n):
        ref = ds_ref[i] + (f64(prior[i]) if accumulate else 0.0)
        if grad == "f32":
            parity.assert_dsrc(f64(dsrc[i]), ref, f"saved dsrc[{i}]")
        else:
            parity.assert_dsrc_bf16(f64(dsrc[i]), ref, f"saved dsrc[{i}]")
    h, al = oracle.forward(s64, f64(q), r, eps)
    parity.assert_dq(f64(dq), dq_ref, parity.dq_bound(s64, f64(q), g64, al, h, r, eps),
                     "saved dq")


def test_backward_saved_full_size_d4096():
    """The backward workload (d = 4096, r = 1024, 10 sources, T = 16384) from saved statistics:
    every source gradient of sampled rows, and dq over all rows, against the oracle."""
    T, d, r, n, eps = 16384, 4096, 1024, 10, 1e-6
    srcs = synth.values(n, T, d, "bf16", 1950, scale=(0.5, 4.0), device="cuda")
    q = synth.queries(1, r, 1.0, seed=1951, device="cuda")[0].contiguous()
    g = synth.upstream(T, d, 1952, device="cuda")
    say("[backward_saved] full size d=4096")
    _, saved = lrar.lrar_forward_save(srcs, q, r, eps)
    dsrc, dq = lrar.lrar_backward_saved(srcs, q, saved, g, r)
    torch.cuda.synchronize()
    rows = torch.as_tensor(np.array(sorted(set([0, T - 1] + list(
        np.random.default_rng(1953).integers(0, T, 30))))), device="cuda")
    s64 = [f64(s.index_select(0, rows)) for s in srcs]
    ds_ref, _ = oracle.backward(s64, f64(q), f64(g.index_select(0, rows)), r, eps)
    for i in range(n):
        parity.assert_dsrc(f64(dsrc[i].index_select(0, rows)), ds_ref[i], f"full dsrc[{i}]")
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
    parity.assert_dq(f64(dq), dq_ref, bound, "full dq")
