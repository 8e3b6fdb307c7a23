"""The calibration streams the bench measures the read against: lrar_mix_stream (the read's
traffic, n bf16 rows in and one out per token) writes the mean of its sources, rounded to bf16,
in every launch shape, over ragged widths and strided rows. Its result is checked against the
mean in float64 (one bf16 rounding plus the float32 sums)."""
import numpy as np
import pytest
import torch

import transformer_depth_wise_lrar_amd as lrar
from gpu_util import f64, needs_gpu, say, sources

pytestmark = [pytest.mark.gpu, needs_gpu]

SHAPES = [(8, 1, 4, 4), (4, 2, 2, 0), (12, 4, 4, 2), (32, 1, 16, 1), (8, 2, 8, 3)]


@pytest.mark.parametrize("T,d,n,ld", [(37, 2056, 3, 2064), (300, 7168, 9, None), (5, 8, 1, None),
                                      (129, 1024, 49, 1032)])
@pytest.mark.parametrize("shape", SHAPES, ids=[f"w{w}-p{p}-s{u}-c{c}" for w, p, u, c in SHAPES])
def test_mix_stream_mean(T, d, n, ld, shape):
    waves, depth, slots, rows = shape
    say(f"mix_stream T={T} d={d} n={n} ld={ld} shape={shape}")
    srcs = sources(n, T, d, "bf16", seed=40 + n, row_stride=ld)
    out = torch.full((T, d + 8), float("nan"), dtype=torch.bfloat16, device="cuda")[:, :d]
    lrar.lrar_mix_stream(srcs, out=out, waves_per_cu=waves, depth=depth, slots=slots,
                         rows_per_wave=rows)
    torch.cuda.synchronize()
    x = np.stack([f64(s) for s in srcs])  # [n, T, d]
    ref = x.mean(axis=0)
    got = f64(out)
    # one bf16 rounding of the float32 sum, plus n float32 roundings of the running sum
    ulp = np.exp2(np.floor(np.log2(np.maximum(np.abs(ref), 1e-30))) - 7)
    bound = ulp + (n + 2) * 2.0 ** -24 * np.abs(x).mean(axis=0)
    assert np.all(np.isfinite(got))
    assert np.all(np.abs(got - ref) <= bound)
