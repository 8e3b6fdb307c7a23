"""Helpers shared by the GPU parity tests: seeded inputs on the device and their exact
float64 copies for the oracle."""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

from transformer_depth_wise_lrar_amd import synth

needs_gpu = pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")


def say(*a):
    """Name the case on stdout before a GPU step (flushed, so a crash still shows it)."""
    print(*a, flush=True)
    sys.stdout.flush()


def sources(n, T, d, io, seed, scale=(0.5, 2.0), row_stride=None, device="cuda"):
    """n sources [T, d] on the device; with row_stride each is a view of a wider buffer."""
    ld = d if row_stride is None else row_stride
    full = synth.values(n, T, ld, io, seed, scale=scale, device="cpu")
    out = []
    for x in full:
        g = x.to(device)
        out.append(g[:, :d] if ld != d else g)
    return out


def f64(t):
    return synth.to_f64(t)


def query(r, seed, std=1.0, device="cuda", nq=1):
    q = synth.queries(nq, r, std, seed, device="cpu").to(device)
    return q[0].contiguous() if nq == 1 else q


def io_of(t):
    return "bf16" if t.dtype == torch.bfloat16 else "f32"


def sample_rows(T, k, seed):
    """Sorted row indices: first, last, a ragged-tail row and k - 3 random rows."""
    rng = np.random.default_rng(seed)
    rows = set([0, T - 1, max(0, T - 3)])
    rows.update(int(x) for x in rng.integers(0, T, size=max(0, k - 3)))
    return np.array(sorted(rows))
