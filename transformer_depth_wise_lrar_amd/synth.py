"""Seeded synthetic inputs for the depth-mix read.

This module draws random tensors and rounds them to the I/O precision; it holds none
of the read's arithmetic. The same tensors feed the HIP library and, decoded to
float64 (an exact conversion), the oracle.

Workloads (shapes and value distributions follow the read sites of the LR-AttnRes
paper's models, §4.1 and App. E; the pages' trained activations and text data are
not available, so independent Gaussian sources stand in for sub-layer outputs, with a
per-source scale that models depth-dependent magnitude):

=====================  ======  =====  =================  =============  ==========
name                   T       d      r                  sources        value dist
=====================  ======  =====  =================  =============  ==========
tiny_f32               64      64     16                 5 (full)       N(0,1) fp32
full_routing_d1024     16384   1024   64                 49 (full)      N(0,1)*U[.5,2] bf16
block_routing_d2048    65536   2048   512 (16/64/2048)   <=10 (blocks)  N(0,1)*U[.5,4] bf16
production_d7168       32768   7168   64 (1792/7168)     <=9 (blocks)   N(0,1)*U[.5,4] bf16
backward_d4096         16384   4096   1024               <=10 (blocks)  N(0,1)*U[.5,4] bf16
=====================  ======  =====  =================  =============  ==========

Queries are fp32 N(0, q_std^2); upstream gradients are fp32 N(0,1).
"""
from __future__ import annotations

import hashlib

import numpy as np
import torch

WORKLOADS = {
    "tiny_f32": dict(T=64, d=64, r=16, eps=1e-6, io="f32", n_sources=5, routing="full",
                     scale=(1.0, 1.0), q_std=0.5),
    "full_routing_d1024": dict(T=8 * 2048, d=1024, r=64, eps=1e-6, io="bf16", n_sources=49,
                               routing="full", scale=(0.5, 2.0), q_std=1.0),
    "block_routing_d2048": dict(T=16 * 4096, d=2048, r=512, r_sweep=(16, 64, 512, 2048),
                                eps=1e-6, io="bf16", n_sources=10, routing="block", M=48, N=8,
                                scale=(0.5, 4.0), q_std=1.0),
    "production_d7168": dict(T=32768, d=7168, r=64, r_sweep=(64, 1792, 7168), eps=1e-6,
                             io="bf16", n_sources=9, routing="block", M=93, N=8,
                             scale=(0.5, 4.0), q_std=1.0),
    "backward_d4096": dict(T=16384, d=4096, r=1024, eps=1e-6, io="bf16", n_sources=10,
                           routing="block", M=48, N=8, scale=(0.5, 4.0), q_std=1.0),
}

TORCH_DTYPE = {"f32": torch.float32, "bf16": torch.bfloat16}


def stream_seed(seed: int, *tags) -> int:
    """A 63-bit seed derived from (seed, tags) so that every tensor has its own stream."""
    h = hashlib.sha256(repr((int(seed),) + tuple(tags)).encode()).digest()
    return int.from_bytes(h[:8], "little") & ((1 << 63) - 1)


def _gen(device, seed, *tags):
    g = torch.Generator(device=device)
    g.manual_seed(stream_seed(seed, *tags))
    return g


def source_scales(n: int, lo: float, hi: float, seed: int) -> np.ndarray:
    """Per-source magnitudes drawn U[lo, hi]."""
    rng = np.random.default_rng(stream_seed(seed, "scales"))
    return rng.uniform(lo, hi, size=n)


def values(n: int, T: int, d: int, io: str, seed: int, scale=(1.0, 1.0), device="cpu",
           row_stride: int | None = None, tag="src"):
    """n source tensors [T, d] of dtype io: N(0,1) times a per-source U[scale] factor,
    rounded to nearest-even in io. With row_stride > d each tensor is a [T, d] view of a
    [T, row_stride] buffer (a strided source)."""
    sc = source_scales(n, scale[0], scale[1], seed)
    ld = d if row_stride is None else row_stride
    out = []
    for i in range(n):
        g = _gen(device, seed, tag, i)
        x = torch.randn((T, ld), generator=g, device=device, dtype=torch.float32)
        x.mul_(float(sc[i]))
        x = x.to(TORCH_DTYPE[io])
        out.append(x[:, :d] if ld != d else x)
    return out


def queries(nq: int, r: int, std: float, seed: int, device="cpu", tag="q"):
    """nq site queries [nq, r], fp32 N(0, std^2)."""
    g = _gen(device, seed, tag)
    return torch.randn((nq, r), generator=g, device=device, dtype=torch.float32) * std


def upstream(T: int, d: int, seed: int, device="cpu", tag="dout"):
    """Upstream gradient dL/dh [T, d], fp32 N(0,1)."""
    g = _gen(device, seed, tag)
    return torch.randn((T, d), generator=g, device=device, dtype=torch.float32)


def to_f64(t: torch.Tensor) -> np.ndarray:
    """Exact float64 copy of a bf16/fp32 tensor (on any device)."""
    return t.detach().to("cpu").to(torch.float64).numpy()
