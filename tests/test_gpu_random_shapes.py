"""Seeded random shapes across the dispatch boundaries of the read and the backward, against the
oracle element by element. The widths straddle the register-tile limits (one to four chunks of 64
units per wave, rows shared by two or four waves, rows past the widest tile), the key widths map to
every spread-piece size, to the row units and to keys that start inside a unit, unaligned widths
and odd row strides take the element path, and every case draws its element type, 1 to 20
sources and 1 to 300 rows (ragged tiles)."""
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
