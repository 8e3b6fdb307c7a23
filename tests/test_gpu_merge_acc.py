"""lrar_merge_accumulate (Phase 2 with the partial-sum update fused in) on the GPU against the
oracle: b_out bit for bit, h with the merge's bar, m' and l' as for lrar_merge."""
import numpy as np
import pytest
import torch

import oracle
import parity
import transformer_depth_wise_lrar_amd as lrar
from gpu_util import f64, needs_gpu, query, say, sources

pytestmark = [pytest.mark.gpu, needs_gpu]

BITS = {"bf16": 8, "f32": 24}


def _case(d, r, io, acc_dtype, with_b, in_place, seed, n_inter=4, T=41):
    """Oracle Phase-1 statistics rounded to their storage types feed both sides; the kernel's
    b_out must equal the oracle's rounded b + o exactly, and h, m', l' meet the merge's bars."""
    inter = sources(n_inter, T, d, io, seed=seed, scale=(0.5, 4.0))
    b, o = sources(2, T, d, io, seed=seed + 1, scale=(0.5, 4.0))
    q = query(r, seed=seed + 2)
    s64 = [f64(s) for s in inter]
    m_o, l_o, acc_o = oracle.stats(s64, f64(q)[None, :], r, 1e-6)
    m = torch.tensor(m_o[0], dtype=torch.float32, device="cuda")
    l = torch.tensor(l_o[0], dtype=torch.float32, device="cuda")
    acc = torch.tensor(acc_o[0], dtype=torch.float32).to(acc_dtype).cuda()
    b64 = f64(b) if with_b else None
    o64 = f64(o)
    say(f"[merge_acc] d={d} r={r} io={io} acc={acc_dtype} b={with_b} in_place={in_place}")
    b_in = b if with_b else None
    b_out = b if (with_b and in_place) else None
    out, b2, m2, l2 = lrar.lrar_merge_accumulate(m, l, acc, b_in, o, q, r, 1e-6, b_out=b_out,
                                                 stats_out=True)
    torch.cuda.synchronize()
    m_in, l_in, acc_in = f64(m), f64(l), f64(acc)
    h_ref, bref, m_ref, l_ref = oracle.merge_accumulate(m_in, l_in, acc_in, b64, o64, f64(q), r,
                                                        1e-6, BITS[io])
    assert np.array_equal(f64(b2), bref), "b_out differs from round(b + o)"
    if in_place and with_b:
        assert b2.data_ptr() == b.data_ptr()
    z_e, _ = oracle.scores([bref], f64(q), r, 1e-6)
    w_extra = np.exp(z_e - m_ref[:, None]) / l_ref[:, None]
    w_prior = l_in * np.exp(m_in - m_ref) / l_ref
    parity.assert_merge(f64(out), h_ref, w_prior, acc_in / l_in[:, None], w_extra, [bref], io,
                        "merge_acc h")
    m2g = f64(m2)
    assert np.all(np.abs(m2g - m_ref) <= 2.0 ** -23 * np.abs(m_ref) + 1e-12)
    l_resc = l_ref * np.exp(m_ref - m2g)
    assert np.all(np.abs(f64(l2) - l_resc) <= 4 * parity.U * l_resc)


@pytest.mark.parametrize("io", ["bf16", "f32"])
@pytest.mark.parametrize("acc_dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("with_b,in_place", [(False, False), (True, False), (True, True)])
def test_merge_accumulate_against_oracle(io, acc_dtype, with_b, in_place):
    _case(1024, 64, io, acc_dtype, with_b, in_place, seed=700)


@pytest.mark.parametrize("d,r", [(64, 16), (513, 64), (2048, 16), (2048, 509), (4096, 1024),
                                 (7168, 1792), (7168, 7168), (16384, 64)])
def test_merge_accumulate_shapes(d, r):
    """One wave per row and four, the element path (d = 513), key widths up to r = d, a key
    whose first unit also holds non-key columns (r = 509)."""
    _case(d, r, "bf16", torch.float32, True, False, seed=710 + d)


def test_merge_accumulate_whole_block_equals_single_pass():
    """Phase 1 over the completed sources, then two writes of the current block through the
    fused update: the second site's h equals one read over the completed sources and the
    stored partial sum, and its stored sum is round(round(o1) + o2)."""
    T, d, r = 64, 1024, 64
    inter = sources(5, T, d, "bf16", seed=720)
    o1, o2 = sources(2, T, d, "bf16", seed=721)
    q1 = query(r, seed=722)
    q2 = query(r, seed=723)
    qs = torch.stack([q1, q2]).contiguous()
    say("[merge_acc] whole block")
    m, l, acc = lrar.lrar_forward_stats(inter, qs, r, 1e-6)
    out1, b = lrar.lrar_merge_accumulate(m[0], l[0], acc[0], None, o1, q1, r, 1e-6)
    out2, b = lrar.lrar_merge_accumulate(m[1], l[1], acc[1], b, o2, q2, r, 1e-6, b_out=b)
    torch.cuda.synchronize()
    s64 = [f64(s) for s in inter]
    b_ref = oracle.round_to_format(f64(o1) + f64(o2), 8)
    assert np.array_equal(f64(b), b_ref)
    h_ref, a_ref = oracle.forward(s64 + [b_ref], f64(q2), r, 1e-6)
    parity.assert_read(f64(out2), h_ref, a_ref, s64 + [b_ref], "bf16", "block site 2")
    h1_ref, a1_ref = oracle.forward(s64 + [f64(o1)], f64(q1), r, 1e-6)
    parity.assert_read(f64(out1), h1_ref, a1_ref, s64 + [f64(o1)], "bf16", "block site 1")


def test_merge_accumulate_full_size_d7168():
    """The production Phase-2 shape: T = 32768, d = 7168, r = 1792, fp32 Phase-1 statistics of 8
    sources; sampled rows against the oracle."""
    from gpu_util import sample_rows
    from transformer_depth_wise_lrar_amd import synth
    T, d, r = 32768, 7168, 1792
    inter = synth.values(8, T, d, "bf16", 730, scale=(0.5, 4.0), device="cuda")
    b, o = synth.values(2, T, d, "bf16", 731, scale=(0.5, 4.0), device="cuda")
    q = synth.queries(1, r, 1.0, seed=732, device="cuda")[0].contiguous()
    say(f"[merge_acc] full size T={T} d={d} r={r}")
    m, l, acc = lrar.lrar_forward_stats(inter, q[None, :].contiguous(), r, 1e-6)
    out, b2 = lrar.lrar_merge_accumulate(m[0], l[0], acc[0], b, o, q, r, 1e-6)
    torch.cuda.synchronize()
    rows = sample_rows(T, 32, seed=733)
    idx = torch.as_tensor(rows, device="cuda")
    pick = lambda t: f64(t.index_select(0, idx))  # noqa: E731
    s64 = [pick(s) for s in inter]
    b_ref = oracle.round_to_format(pick(b) + pick(o), 8)
    assert np.array_equal(pick(b2), b_ref)
    h_ref, a_ref = oracle.forward(s64 + [b_ref], f64(q), r, 1e-6)
    parity.assert_read(pick(out), h_ref, a_ref, s64 + [b_ref], "bf16", "full size h")
