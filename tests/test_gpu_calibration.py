"""The calibration streams the bench measures the kernels against: lrar_mix_stream (n bf16 rows
in and nout rows out per token: one bf16 output is a read's traffic, several or float32 ones
the write-heavy mixes of Phase 1 and the backward) writes the mean of its sources to every
output, in every launch shape, over ragged widths and strided rows. The result is checked
against the mean in float64 (the float32 sums, plus one bf16 rounding for bf16 outputs)."""
import numpy as np
import pytest
import torch

import transformer_depth_wise_lrar_amd as lrar
from gpu_util import f64, needs_gpu, say, sources

pytestmark = [pytest.mark.gpu, needs_gpu]

# (waves per CU, sources loaded together, units a lane, rows per row group per launch,
# lockstep, waves per row)
SHAPES = [(8, 1, 4, 4, 0, 1), (4, 2, 2, 0, 1, 1), (12, 4, 4, 2, 2, 1), (32, 1, 16, 1, 1, 1),
          (8, 2, 8, 3, 2, 1), (8, 1, 4, 2, 1, 4), (12, 2, 2, 0, 2, 2), (16, 1, 8, 3, 0, 4)]
SHAPE_IDS = [f"w{w}-p{p}-s{u}-c{c}-l{k}-r{g}" for w, p, u, c, k, g in SHAPES]


def check_mean(srcs, outs, bf16):
    x = np.stack([f64(s) for s in srcs])  # [n, T, d]
    n = len(srcs)
    ref = x.mean(axis=0)
    # n float32 roundings of the running sum (and of w = 1/n), plus one bf16 rounding
    bound = (n + 2) * 2.0 ** -24 * np.abs(x).mean(axis=0)
    if bf16:
        bound = bound + np.exp2(np.floor(np.log2(np.maximum(np.abs(ref), 1e-30))) - 7)
    for j, o in enumerate(outs):
        got = f64(o)
        assert np.all(np.isfinite(got)), f"out[{j}]"
        assert np.all(np.abs(got - ref) <= bound), f"out[{j}]"


@pytest.mark.parametrize("T,d,n,ld", [(37, 2056, 3, 2064), (300, 7168, 9, None), (5, 8, 1, None),
                                      (129, 1024, 49, 1032)])
@pytest.mark.parametrize("shape", SHAPES, ids=SHAPE_IDS)
def test_mix_stream_mean(T, d, n, ld, shape):
    waves, depth, slots, rows, lock, wpr = shape
    say(f"mix_stream T={T} d={d} n={n} ld={ld} shape={shape}")
    srcs = sources(n, T, d, "bf16", seed=40 + n, row_stride=ld)
    out = torch.full((T, d + 8), float("nan"), dtype=torch.bfloat16, device="cuda")[:, :d]
    lrar.lrar_mix_stream(srcs, out=out, waves_per_cu=waves, depth=depth, slots=slots,
                         rows_per_wave=rows, lockstep=lock, waves_per_row=wpr)
    torch.cuda.synchronize()
    check_mean(srcs, [out], True)


@pytest.mark.parametrize("T,d,n,nout,dt", [(300, 7168, 8, 12, "f32"), (300, 7168, 8, 12, "bf16"),
                                           (61, 4096, 12, 10, "f32"), (33, 2056, 3, 1, "f32"),
                                           (17, 1032, 4, 2, "bf16")])
@pytest.mark.parametrize("shape", SHAPES[:3] + SHAPES[5:7], ids=SHAPE_IDS[:3] + SHAPE_IDS[5:7])
def test_mix_stream_outputs(T, d, n, nout, dt, shape):
    """Several outputs (of Phase 1's and the backward's mixes), float32 or bf16, some strided."""
    waves, depth, slots, rows, lock, wpr = shape
    say(f"mix_stream outputs T={T} d={d} n={n} nout={nout} {dt} shape={shape}")
    srcs = sources(n, T, d, "bf16", seed=60 + n)
    tdt = torch.float32 if dt == "f32" else torch.bfloat16
    outs = [torch.full((T, d + 8 * (j % 2)), float("nan"), dtype=tdt, device="cuda")[:, :d]
            for j in range(nout)]
    lrar.lrar_mix_stream(srcs, out=outs, waves_per_cu=waves, depth=depth, slots=slots,
                         rows_per_wave=rows, lockstep=lock, waves_per_row=wpr)
    torch.cuda.synchronize()
    check_mean(srcs, outs, dt == "bf16")
