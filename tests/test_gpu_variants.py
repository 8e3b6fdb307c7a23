"""The full-width-RMS control read (lrar_forward_fullrms) and the separate-key read
(lrar_forward_keys) on the GPU against the oracle, element by element, with the same bars as
lrar_forward."""
import math

import numpy as np
import pytest
import torch

import oracle
import parity
import transformer_depth_wise_lrar_amd as lrar
from gpu_util import f64, io_of, needs_gpu, query, sample_rows, say, sources
from transformer_depth_wise_lrar_amd import synth

pytestmark = [pytest.mark.gpu, needs_gpu]

DT = {"f32": torch.float32, "bf16": torch.bfloat16}


def check_fullrms(srcs, q, r, eps, where):
    say(f"[fullrms] {where} T={srcs[0].shape[0]} d={srcs[0].shape[1]} r={r} n={len(srcs)} "
        f"io={io_of(srcs[0])}")
    out, alpha = lrar.lrar_forward_fullrms(srcs, q, r, eps, alpha=True)
    torch.cuda.synchronize()
    s64 = [f64(s) for s in srcs]
    h_ref, a_ref = oracle.forward_fullrms(s64, f64(q), r, eps)
    parity.assert_weights(f64(alpha), a_ref, where + " alpha")
    parity.assert_read(f64(out), h_ref, a_ref, s64, io_of(srcs[0]), where + " h")
    return out, alpha


def check_keys(srcs, keys, q, r, eps, where):
    say(f"[keys] {where} T={srcs[0].shape[0]} d={srcs[0].shape[1]} r={r} n={len(srcs)} "
        f"io={io_of(srcs[0])} key_ld={keys[0].stride(0)}")
    out, alpha = lrar.lrar_forward_keys(srcs, keys, q, r, eps, alpha=True)
    torch.cuda.synchronize()
    s64 = [f64(s) for s in srcs]
    h_ref, a_ref = oracle.forward_keys(s64, [f64(k) for k in keys], f64(q), r, eps)
    parity.assert_weights(f64(alpha), a_ref, where + " alpha")
    parity.assert_read(f64(out), h_ref, a_ref, s64, io_of(srcs[0]), where + " h")
    return out, alpha


def key_tensors(n, T, r, io, seed, key_ld=None, offset=0):
    """n keys [T, r]; with key_ld each is a view of a wider buffer, starting `offset`
    elements in (so its rows need not be 16-byte aligned)."""
    ld = r if key_ld is None else key_ld
    full = synth.values(n, T, ld + offset, io, seed, scale=(0.5, 2.0), device="cuda", )
    return [x[:, offset:offset + r] for x in full]


# ---- the full-width-RMS control read ---------------------------------------------------------

@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_fullrms_closed_form(io):
    """The pinned closed form: o_A = (1,1,1,1) and o_B = (2,0,0,0) have full RMS 1, so with
    q = (ln 3, 0) the weights are (3/4, 1/4) and h = (5/4, 3/4, 3/4, 3/4)."""
    dt = DT[io]
    oA = torch.tensor([[1.0, 1.0, 1.0, 1.0]], dtype=dt, device="cuda")
    oB = torch.tensor([[2.0, 0.0, 0.0, 0.0]], dtype=dt, device="cuda")
    q = torch.tensor([math.log(3.0), 0.0], dtype=torch.float32, device="cuda")
    say(f"[fullrms] closed form io={io}")
    out, al = lrar.lrar_forward_fullrms([oA, oB], q, 2, 0.0, alpha=True)
    torch.cuda.synchronize()
    assert np.allclose(f64(al)[0], [0.75, 0.25], rtol=0, atol=1e-7)
    assert np.allclose(f64(out)[0], [1.25, 0.75, 0.75, 0.75], rtol=0, atol=1e-6)


@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("d,r", [(64, 16), (1024, 64), (1024, 1000), (1024, 1001), (513, 64),
                                 (2048, 512), (2048, 509), (4096, 1024), (7168, 1792)])
def test_fullrms_shapes(io, d, r):
    """One wave per row (d up to 4 chunks) and four waves per row, the element path (d = 513),
    keys of every width, keys whose first unit also holds non-key columns (r = 1001, 509);
    ragged row count."""
    srcs = sources(10, 77, d, io, seed=600 + d + r, scale=(0.5, 4.0))
    q = query(r, seed=601)
    for n in (1, 3, 10):
        check_fullrms(srcs[:n], q, r, 1e-6, f"d={d} r={r} n={n}")


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_fullrms_r_equals_d_is_standard_attnres(io):
    """At r = d the control read is standard AttnRes (oracle.attnres_standard)."""
    d = 256
    srcs = sources(6, 33, d, io, seed=610)
    q = query(d, seed=611, std=0.2)
    say(f"[fullrms] r = d = {d} io={io}")
    out, al = lrar.lrar_forward_fullrms(srcs, q, d, 1e-6, alpha=True)
    torch.cuda.synchronize()
    s64 = [f64(s) for s in srcs]
    h_ref, a_ref = oracle.attnres_standard(s64, f64(q), 1e-6)
    parity.assert_weights(f64(al), a_ref, "r=d alpha")
    parity.assert_read(f64(out), h_ref, a_ref, s64, io, "r=d h")


def test_fullrms_widest_row():
    srcs = sources(3, 9, 16384, "bf16", seed=612, scale=(0.5, 4.0))
    check_fullrms(srcs, query(64, seed=613), 64, 1e-6, "d=16384")


def test_fullrms_full_size_d1024():
    """The full-routing shape (T = 16384, d = 1024, r = 64, 49 sources) on sampled rows."""
    T, d, r, n = 8 * 2048, 1024, 64, 49
    srcs = synth.values(n, T, d, "bf16", 620, scale=(0.5, 2.0), device="cuda")
    q = synth.queries(1, r, 1.0, seed=621, device="cuda")[0].contiguous()
    say(f"[fullrms] full size T={T} d={d} r={r} n={n}")
    out, alpha = lrar.lrar_forward_fullrms(srcs, q, r, 1e-6, alpha=True)
    torch.cuda.synchronize()
    rows = sample_rows(T, 48, seed=622)
    idx = torch.as_tensor(rows, device="cuda")
    s64 = [f64(s.index_select(0, idx)) for s in srcs]
    h_ref, a_ref = oracle.forward_fullrms(s64, f64(q), r, 1e-6)
    parity.assert_weights(f64(alpha.index_select(0, idx)), a_ref, "full size alpha")
    parity.assert_read(f64(out.index_select(0, idx)), h_ref, a_ref, s64, "bf16", "full size h")


# ---- the separate-key read -------------------------------------------------------------------

@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_keys_worked_example(io):
    """The worked example with the keys (1, 0) and (0, 1) held apart from the values: weights
    (3/4, 1/4) whatever the values hold."""
    dt = DT[io]
    kA = torch.tensor([[1.0, 0.0]], dtype=dt, device="cuda")
    kB = torch.tensor([[0.0, 1.0]], dtype=dt, device="cuda")
    oA = torch.tensor([[4.0, -1.0, 7.0, -2.0]], dtype=dt, device="cuda")
    oB = torch.tensor([[0.0, 3.0, 5.0, 3.0]], dtype=dt, device="cuda")
    q = torch.tensor([math.log(3.0) / math.sqrt(2.0), 0.0], dtype=torch.float32, device="cuda")
    say(f"[keys] worked example io={io}")
    out, al = lrar.lrar_forward_keys([oA, oB], [kA, kB], q, 2, 0.0, alpha=True)
    torch.cuda.synchronize()
    assert np.allclose(f64(al)[0], [0.75, 0.25], rtol=0, atol=1e-7)
    want = 0.75 * f64(oA)[0] + 0.25 * f64(oB)[0]
    assert np.allclose(f64(out)[0], want, rtol=0, atol=1e-6 if io == "f32" else 4e-2)


@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("r", [1, 16, 32, 33, 64, 96, 100, 128, 200, 256, 384, 512])
def test_keys_ranks(io, r):
    """Every spread key piece (1 to 8 elements per lane, row-local or over all lanes), with key
    rows packed (stride r) and strided (stride r + 8); ragged row count."""
    d = 1024
    srcs = sources(10, 77, d, io, seed=630 + r, scale=(0.5, 4.0))
    q = query(r, seed=631)
    for key_ld in (r, r + 8):
        keys = key_tensors(10, 77, r, io, seed=632 + r, key_ld=key_ld)
        for n in (1, 3, 10):
            check_keys(srcs[:n], keys[:n], q, r, 1e-6, f"r={r} key_ld={key_ld} n={n}")


@pytest.mark.parametrize("io,d,r", [(io, d, r) for io in ("f32", "bf16")
                                     for d, r in ((64, 16), (513, 64), (2048, 32), (4096, 64))]
                         + [("f32", 8192, 128), ("bf16", 16384, 128)])
def test_keys_widths(io, d, r):
    """Value rows of every tile shape up to the widest (32 chunks), the element path
    (d = 513) and misaligned key rows (each key starts one element into its buffer, so only
    single-element pieces fit)."""
    srcs = sources(9, 45, d, io, seed=640 + d, scale=(0.5, 4.0))
    q = query(r, seed=641)
    keys = key_tensors(9, 45, r, io, seed=642 + d)
    check_keys(srcs, keys, q, r, 1e-6, f"d={d} r={r}")
    if r <= 64:
        keys = key_tensors(9, 45, r, io, seed=643 + d, key_ld=r + 1, offset=1)
        check_keys(srcs, keys, q, r, 1e-6, f"d={d} r={r} misaligned keys")


def test_keys_equal_value_tails_match_slice_read():
    """Keys copied from the values' last r columns: the separate-key read and the sliced read
    both meet the oracle's sliced read (LR-AttnRes paper App. C.1: a key taken from the value's
    own tail is the sliced key)."""
    T, d, r = 50, 1024, 64
    srcs = sources(7, T, d, "bf16", seed=650)
    keys = [s[:, d - r:].contiguous() for s in srcs]
    q = query(r, seed=651)
    say("[keys] keys = value tails")
    o1, a1 = lrar.lrar_forward_keys(srcs, keys, q, r, 1e-6, alpha=True)
    o2, a2 = lrar.lrar_forward(srcs, q, r, 1e-6, alpha=True)
    torch.cuda.synchronize()
    s64 = [f64(s) for s in srcs]
    h_ref, a_ref = oracle.forward(s64, f64(q), r, 1e-6)
    for name, o, a in (("keys", o1, a1), ("slice", o2, a2)):
        parity.assert_weights(f64(a), a_ref, f"{name} read vs oracle slice alpha")
        parity.assert_read(f64(o), h_ref, a_ref, s64, "bf16", f"{name} read vs oracle slice h")


def test_keys_wide_rank_takes_the_chunked_read():
    """r = 1000 is wider than a spread key piece reaches: the column-chunked read serves it."""
    srcs = sources(3, 8, 1024, "bf16", seed=660)
    keys = key_tensors(3, 8, 1000, "bf16", seed=661)
    check_keys(srcs, keys, query(1000, seed=662), 1000, 1e-6, "r=1000")


def test_keys_full_size_d1024():
    """The pages' projected-key shape: d = 1024, r = 32, 49 sources, T = 16384, sampled rows."""
    T, d, r, n = 8 * 2048, 1024, 32, 49
    srcs = synth.values(n, T, d, "bf16", 670, scale=(0.5, 2.0), device="cuda")
    keys = synth.values(n, T, r, "bf16", 671, scale=(0.5, 2.0), device="cuda")
    q = synth.queries(1, r, 1.0, seed=672, device="cuda")[0].contiguous()
    say(f"[keys] full size T={T} d={d} r={r} n={n}")
    out, alpha = lrar.lrar_forward_keys(srcs, keys, q, r, 1e-6, alpha=True)
    torch.cuda.synchronize()
    rows = sample_rows(T, 48, seed=673)
    idx = torch.as_tensor(rows, device="cuda")
    s64 = [f64(s.index_select(0, idx)) for s in srcs]
    k64 = [f64(k.index_select(0, idx)) for k in keys]
    h_ref, a_ref = oracle.forward_keys(s64, k64, f64(q), r, 1e-6)
    parity.assert_weights(f64(alpha.index_select(0, idx)), a_ref, "full size alpha")
    parity.assert_read(f64(out.index_select(0, idx)), h_ref, a_ref, s64, "bf16", "full size h")
