"""lrar_forward on the GPU against the oracle (element by element)."""
import math

import numpy as np
import pytest
import torch

import oracle
import parity
import transformer_depth_wise_lrar_amd as lrar
from gpu_util import f64, io_of, needs_gpu, query, say, sources

pytestmark = [pytest.mark.gpu, needs_gpu]

VARIANTS = ["two_pass", "online", "auto"]


def run_and_check(srcs, q, r, eps, variant, where):
    say(f"[read] {where} variant={variant} T={srcs[0].shape[0]} d={srcs[0].shape[1]} r={r} "
        f"n={len(srcs)} io={io_of(srcs[0])}")
    out, alpha = lrar.lrar_forward(srcs, q, r, eps, alpha=True, variant=variant)
    torch.cuda.synchronize()
    s64 = [f64(s) for s in srcs]
    h_ref, a_ref = oracle.forward(s64, f64(q), r, eps)
    parity.assert_weights(f64(alpha), a_ref, where + " alpha")
    parity.assert_read(f64(out), h_ref, a_ref, s64, io_of(srcs[0]), where + " h")
    return out, alpha


@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("variant", VARIANTS)
def test_worked_example(io, variant):
    """The explainer's four-number example on the device: weights (3/4, 1/4), output
    coordinate 1 moves from 3 to 6 when o_A's first coordinate moves from 4 to 8."""
    dt = torch.float32 if io == "f32" else torch.bfloat16
    q = torch.tensor([math.log(3.0) / math.sqrt(2.0), 0.0], dtype=torch.float32, device="cuda")
    for a, b in [(0.0, 0.0), (1.0, -2.0), (-2.0, 1.0)]:
        oA = torch.tensor([[4.0, a, 1.0, 0.0]], dtype=dt, device="cuda")
        oB = torch.tensor([[0.0, b, 0.0, 1.0]], dtype=dt, device="cuda")
        out, al = lrar.lrar_forward([oA, oB], q, 2, 0.0, alpha=True, variant=variant)
        torch.cuda.synchronize()
        assert np.allclose(f64(al)[0], [0.75, 0.25], rtol=0, atol=1e-6)
        h = f64(out)[0]
        assert abs(h[0] - 3.0) < 1e-5 and abs(h[2] - 0.75) < 1e-6 and abs(h[3] - 0.25) < 1e-6
        assert abs(h[1] - (0.75 * a + 0.25 * b)) < 1e-5
        oA[0, 0] = 8.0
        out2, al2 = lrar.lrar_forward([oA, oB], q, 2, 0.0, alpha=True, variant=variant)
        torch.cuda.synchronize()
        assert torch.equal(al, al2)
        assert abs(f64(out2)[0][0] - 6.0) < 1e-5


@pytest.mark.parametrize("variant", VARIANTS)
def test_tiny_full_routing_all_sites(variant):
    """The tiny fp32 workload: T=64, d=64, r=16, five sources, every read site in order."""
    T, d, r, eps = 64, 64, 16, 1e-6
    srcs = sources(5, T, d, "f32", seed=11, scale=(1.0, 1.0))
    qs = query(r, seed=12, std=0.5, nq=5)
    for n in range(1, 6):
        run_and_check(srcs[:n], qs[n - 1].contiguous(), r, eps, variant, f"tiny site n={n}")


@pytest.mark.parametrize("variant", VARIANTS)
@pytest.mark.parametrize("n", [1, 2, 13, 49])
@pytest.mark.parametrize("qstd", [1.0, 0.125])
def test_full_routing_width_1024(variant, n, qstd):
    """d=1024, r=64, bf16, T=301 rows (several workgroups and a ragged last one); a sharp
    (q ~ N(0,1)) and a soft (q ~ N(0, 1/r)) routing distribution."""
    srcs = sources(n, 301, 1024, "bf16", seed=20 + n)
    q = query(64, seed=21, std=qstd)
    run_and_check(srcs, q, 64, 1e-6, variant, f"d1024 n={n} qstd={qstd}")


@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("r", [1, 64, 384, 513])
@pytest.mark.parametrize("n", [1, 2, 5, 9, 10])
def test_unaligned_width_513(io, r, n):
    """Unaligned width d=513 (scalar path) with every key width from 1 to d."""
    srcs = sources(n, 37, 513, io, seed=30 + n)
    q = query(r, seed=31)
    for variant in VARIANTS:
        run_and_check(srcs, q, r, 1e-6, variant, f"d513 r={r}")


@pytest.mark.parametrize("d,r", [(1536, 384), (2560, 640), (2048, 16), (2048, 512),
                                 (2048, 2048), (4096, 1024), (7168, 64), (7168, 1792)])
@pytest.mark.parametrize("n", [2, 5, 9, 10])
def test_non_power_of_two_ranks(d, r, n):
    """Key widths 384 and 640 at the 1B/4B model widths, and the other workload shapes."""
    srcs = sources(n, 19, d, "bf16", seed=40 + n, scale=(0.5, 4.0))
    q = query(r, seed=41)
    for variant in VARIANTS:
        run_and_check(srcs, q, r, 1e-6, variant, f"d{d} r={r}")


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_repeated_and_strided_sources(io):
    """Repeated sources (one buffer several times), row-strided sources that keep 16-byte
    alignment (vector path) or break it (scalar path), and a strided query row."""
    d, r, T = 1024, 64, 77
    base = sources(3, T, d, io, seed=50)
    wide = sources(2, T, d, io, seed=51, row_stride=d + 8)
    odd = sources(2, T, d, io, seed=52, row_stride=d + 3)
    Q = torch.randn((3, r + 5), generator=torch.Generator().manual_seed(53)).cuda()
    q = Q[1, :r]
    for name, srcs in [("repeated", [base[0], base[1], base[0], base[0]]),
                       ("strided16", wide + [base[2]]),
                       ("strided_odd", odd + [base[1]])]:
        for variant in VARIANTS:
            run_and_check(srcs, q, r, 1e-6, variant, name)


def test_changed_input_replay():
    """The same buffers read again after their contents change in place."""
    srcs = sources(5, 64, 2048, "bf16", seed=60, scale=(0.5, 4.0))
    q = query(512, seed=61)
    out1, _ = run_and_check(srcs, q, 512, 1e-6, "auto", "replay 1")
    keep = out1.clone()
    srcs[2].mul_(-3.0)
    srcs[4][:, -512:] = 0.5
    out2, _ = run_and_check(srcs, q, 512, 1e-6, "auto", "replay 2")
    assert not torch.equal(keep, out2)


@pytest.mark.parametrize("variant", ["two_pass", "online"])
def test_deterministic(variant):
    srcs = sources(9, 129, 2048, "bf16", seed=70, scale=(0.5, 4.0))
    q = query(512, seed=71)
    a, al = lrar.lrar_forward(srcs, q, 512, 1e-6, alpha=True, variant=variant)
    b, bl = lrar.lrar_forward(srcs, q, 512, 1e-6, alpha=True, variant=variant)
    torch.cuda.synchronize()
    assert torch.equal(a, b) and torch.equal(al, bl)


def test_single_source_is_identity():
    srcs = sources(1, 50, 1024, "bf16", seed=80)
    out, al = lrar.lrar_forward(srcs, query(64, seed=81), 64, 1e-6, alpha=True)
    torch.cuda.synchronize()
    assert torch.equal(out, srcs[0]) and torch.all(al == 1.0)


def test_zero_query_uniform_mean():
    srcs = sources(6, 40, 1024, "f32", seed=82)
    q = torch.zeros(64, dtype=torch.float32, device="cuda")
    out, al = lrar.lrar_forward(srcs, q, 64, 1e-6, alpha=True)
    torch.cuda.synchronize()
    assert torch.allclose(al, torch.full_like(al, 1 / 6), rtol=0, atol=1e-7)
    mean = sum(f64(s) for s in srcs) / 6
    assert np.abs(f64(out) - mean).max() <= 1e-5 * max(np.abs(f64(s)).max() for s in srcs)


def test_zero_slice_with_zero_eps_gives_nan():
    """eps = 0 and an all-zero key slice: 0/0, so that token's output is NaN (as in the
    oracle); other tokens are unaffected."""
    srcs = sources(2, 8, 64, "f32", seed=83)
    srcs[0][3, -16:] = 0.0
    out, al = lrar.lrar_forward(srcs, query(16, seed=84), 16, 0.0, alpha=True)
    torch.cuda.synchronize()
    o = f64(out)
    assert np.isnan(o[3]).all() and np.isfinite(np.delete(o, 3, axis=0)).all()


def test_empty_batch():
    srcs = [torch.empty((0, 1024), dtype=torch.bfloat16, device="cuda")] * 2
    out, al = lrar.lrar_forward(srcs, query(64, seed=85), 64, 1e-6, alpha=True)
    torch.cuda.synchronize()
    assert out.shape == (0, 1024)


@pytest.mark.parametrize("io", ["bf16", "f32"])
@pytest.mark.parametrize("r", [1, 16, 63, 64, 65, 100, 127, 128, 129, 200, 254, 256, 257, 384,
                               512, 1000, 1024])
def test_key_paths(io, r):
    """Every way the key is scored: spread pieces of 1, 2 or 4 elements per lane (r up to 64,
    128, 256 when the key start allows), key units in the last slot or in every slot; on a
    ragged row count so the last tile is partial."""
    srcs = sources(10, 77, 1024, io, seed=90 + r)
    q = query(r, seed=91)
    for n in (3, 10):
        for variant in VARIANTS:
            run_and_check(srcs[:n], q, r, 1e-6, variant, f"key path r={r} n={n}")


@pytest.mark.parametrize("d,r,io", [(4096, 512, "f32"), (8192, 8192, "f32"), (12288, 64, "bf16"),
                                    (12288, 3000, "bf16"), (16384, 16384, "bf16")])
def test_wide_rows(d, r, io):
    """Rows shared by the four waves of a workgroup, up to the widest tile (32 chunks), for
    every variant and the merge."""
    srcs = sources(4, 21, d, io, seed=95, scale=(0.5, 4.0))
    q = query(r, seed=96)
    for variant in VARIANTS:
        run_and_check(srcs, q, r, 1e-6, variant, f"wide d{d} r={r}")
