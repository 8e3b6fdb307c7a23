"""The largest counts the boundary accepts: 64 sources (LRAR_MAX_SOURCES) for every read and
the backward, 64 site queries (LRAR_MAX_QUERIES) for Phase 1 on both of its kernels, against
the oracle with the usual bars."""
import numpy as np
import pytest
import torch

import oracle
import parity
import transformer_depth_wise_lrar_amd as lrar
from gpu_util import f64, needs_gpu, query, say, sources
from transformer_depth_wise_lrar_amd import synth

pytestmark = [pytest.mark.gpu, needs_gpu]

N = lrar.MAX_SOURCES
NQ = lrar.MAX_QUERIES


@pytest.fixture(scope="module")
def srcs64():
    return sources(N, 19, 1024, "bf16", seed=900, scale=(0.5, 2.0))


@pytest.mark.parametrize("variant", ["two_pass", "online"])
def test_forward_64_sources(srcs64, variant):
    q = query(64, seed=901)
    say(f"[limits] forward n={N} {variant}")
    out, al = lrar.lrar_forward(srcs64, q, 64, 1e-6, alpha=True, variant=variant)
    torch.cuda.synchronize()
    s64 = [f64(s) for s in srcs64]
    h_ref, a_ref = oracle.forward(s64, f64(q), 64, 1e-6)
    parity.assert_weights(f64(al), a_ref, "alpha")
    parity.assert_read(f64(out), h_ref, a_ref, s64, "bf16", "h")


def test_control_and_separate_keys_64_sources(srcs64):
    q = query(32, seed=902)
    keys = synth.values(N, 19, 32, "bf16", 903, scale=(0.5, 2.0), device="cuda")
    say(f"[limits] fullrms and keys n={N}")
    out, al = lrar.lrar_forward_fullrms(srcs64, q, 32, 1e-6, alpha=True)
    out2, al2 = lrar.lrar_forward_keys(srcs64, keys, q, 32, 1e-6, alpha=True)
    torch.cuda.synchronize()
    s64 = [f64(s) for s in srcs64]
    h_ref, a_ref = oracle.forward_fullrms(s64, f64(q), 32, 1e-6)
    parity.assert_weights(f64(al), a_ref, "fullrms alpha")
    parity.assert_read(f64(out), h_ref, a_ref, s64, "bf16", "fullrms h")
    h2, a2 = oracle.forward_keys(s64, [f64(k) for k in keys], f64(q), 32, 1e-6)
    parity.assert_weights(f64(al2), a2, "keys alpha")
    parity.assert_read(f64(out2), h2, a2, s64, "bf16", "keys h")


def test_merge_64_extra_sources(srcs64):
    """Phase-1 statistics of two sources merged with 62 more."""
    q = query(64, seed=904)
    say(f"[limits] merge with {N - 2} extra sources")
    m, l, acc = lrar.lrar_forward_stats(srcs64[:2], q[None, :].contiguous(), 64, 1e-6)
    out = lrar.lrar_merge(m[0], l[0], acc[0], srcs64[2:], q, 64, 1e-6)
    torch.cuda.synchronize()
    s64 = [f64(s) for s in srcs64]
    h_ref, a_ref = oracle.forward(s64, f64(q), 64, 1e-6)
    parity.assert_read(f64(out), h_ref, a_ref, s64, "bf16", "two-phase h")


def test_backward_64_sources(srcs64):
    q = query(64, seed=905)
    dout = synth.upstream(19, 1024, 906, device="cpu").cuda()
    say(f"[limits] backward n={N}")
    dsrc, dq = lrar.lrar_backward(srcs64, q, dout, 64, 1e-6)
    torch.cuda.synchronize()
    s64 = [f64(s) for s in srcs64]
    g64 = f64(dout)
    ds_ref, dq_ref = oracle.backward(s64, f64(q), g64, 64, 1e-6)
    for i in range(N):
        parity.assert_dsrc(f64(dsrc[i]), ds_ref[i], f"dsrc[{i}]")
    h, al = oracle.forward(s64, f64(q), 64, 1e-6)
    parity.assert_dq(f64(dq), dq_ref, parity.dq_bound(s64, f64(q), g64, al, h, 64, 1e-6))


@pytest.mark.parametrize("n", [8, 9])
def test_stats_64_queries(srcs64, n):
    """64 queries in one call: in groups of 12 on the workgroup kernel (n = 8), and on the
    one-wave-per-row kernel (n = 9, more sources than the workgroup kernel takes)."""
    qs = query(64, seed=907, nq=NQ)
    say(f"[limits] stats nq={NQ} n={n}")
    m, l, acc = lrar.lrar_forward_stats(srcs64[:n], qs, 64, 1e-6)
    torch.cuda.synchronize()
    s64 = [f64(s) for s in srcs64[:n]]
    q64 = f64(qs)
    m_o, l_o, acc_o = oracle.stats(s64, q64, 64, 1e-6)
    for s in range(NQ):
        z_o, _ = oracle.scores(s64, q64[s], 64, 1e-6)
        parity.assert_stats(f64(m[s]), f64(l[s]), f64(acc[s]), m_o[s], l_o[s], acc_o[s], z_o,
                            s64, "f32", f"query {s}")
