"""Pins that tie the oracle to facts fixed by the pages and by mathematics.

Each pin takes an ``oracle.Oracle`` and raises AssertionError on a mismatch. They are
run against the real oracle (test_oracle_pins.py) and against deliberately broken copies
of it (test_oracle_mutants.py), which must each fail at least one pin.

Citations name the public pages:
  [Explainer] "Low-Rank Attention Residuals", the author's explainer page.
  [Paper]     "Low-Rank Attention Residuals" (J. Su), the paper's HTML version.
  [AttnRes-TR] "Attention Residuals (AttnRes / Block AttnRes) - Technical Report" summary.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _rng(seed):
    return np.random.default_rng(seed)


def _rand_sources(rng, n, T, d, scale=1.0):
    return [rng.standard_normal((T, d)) * scale * rng.uniform(0.5, 2.0) for _ in range(n)]


def _worked():
    with open(os.path.join(GOLDEN, "worked_example.json")) as f:
        return json.load(f)


# --- a1-a5: the read --------------------------------------------------------------------

def pin_worked_example(orc):
    """[Explainer] 'A complete four-number example': weights (3/4, 1/4); output coordinate 1
    is 3 and becomes 6 when o_A's first coordinate goes from 4 to 8; weights unchanged.
    Run at eps = 0 because the page ignores epsilon."""
    g = _worked()
    q = np.array([math.log(3.0) / math.sqrt(2.0), 0.0])
    for a in g["free_values"]:
        for b in g["free_values"]:
            oA = np.array([[4.0, a, 1.0, 0.0]])
            oB = np.array([[0.0, b, 0.0, 1.0]])
            h, al = orc.forward([oA, oB], q, 2, 0.0)
            assert np.allclose(al[0], g["expected_weights"], rtol=0, atol=1e-15), al
            assert abs(h[0, 0] - g["expected_h_coord1"]) < 1e-14, h
            assert abs(h[0, 1] - (0.75 * a + 0.25 * b)) < 1e-14, h
            assert abs(h[0, 2] - 0.75) < 1e-15 and abs(h[0, 3] - 0.25) < 1e-15, h
            z, rho = orc.scores([oA, oB], q, 2, 0.0)
            assert abs(z[0, 0] - math.log(3.0)) < 1e-15 and abs(z[0, 1]) < 1e-15, z
            # RMS of (1,0) is 1/sqrt2, so the normalised key is (sqrt2, 0)
            assert np.allclose(rho[0], [1 / math.sqrt(2.0)] * 2, rtol=0, atol=1e-15), rho
            oA2 = oA.copy()
            oA2[0, 0] = g["edit"]["o_A_coord1_to"]
            h2, al2 = orc.forward([oA2, oB], q, 2, 0.0)
            assert np.array_equal(al2, al), (al, al2)
            assert abs(h2[0, 0] - g["edit"]["expected_h_coord1"]) < 1e-14, h2


def pin_eps_placement(orc):
    """Where epsilon goes (reading of [Explainer] code `rms`: eps is added to the mean of
    squares, inside the square root). With the worked example's keys the mean of squares is
    1/2; eps = 1/2 then makes the RMS exactly 1, so q = (log 3, 0) must give (3/4, 1/4).
    Any other placement (outside the root, added to the sum, dropped) changes the weights."""
    q = np.array([math.log(3.0), 0.0])
    oA = np.array([[4.0, 7.0, 1.0, 0.0]])
    oB = np.array([[0.0, -3.0, 0.0, 1.0]])
    h, al = orc.forward([oA, oB], q, 2, 0.5)
    assert np.allclose(al[0], [0.75, 0.25], rtol=0, atol=1e-15), al
    z, rho = orc.scores([oA, oB], q, 2, 0.5)
    assert np.allclose(rho[0], [1.0, 1.0], rtol=0, atol=1e-15), rho


def pin_zero_query_uniform(orc):
    """[Explainer] 'A short description...': zero queries give uniform source weights, so the
    read is the plain mean of the sources."""
    rng = _rng(1)
    for n in (1, 2, 5, 9):
        srcs = _rand_sources(rng, n, 7, 12)
        h, al = orc.forward(srcs, np.zeros(5), 5, 1e-6)
        assert np.allclose(al, 1.0 / n, rtol=0, atol=1e-15), al
        mean = sum(srcs) / n
        assert np.allclose(h, mean, rtol=1e-14, atol=1e-14)


def pin_weights_simplex(orc):
    """[Explainer]: softmax turns scores into positive weights summing to one; [Paper] §3.1:
    the softmax runs over the sources, independently per token."""
    rng = _rng(2)
    srcs = _rand_sources(rng, 6, 33, 20)
    q = rng.standard_normal(8) * 2
    h, al = orc.forward(srcs, q, 8, 1e-6)
    assert np.all(al > 0)
    assert np.allclose(al.sum(axis=1), 1.0, rtol=0, atol=1e-14)
    # token independence: a read over one row alone gives the same row
    for t in (0, 17, 32):
        h1, al1 = orc.forward([s[t:t + 1] for s in srcs], q, 8, 1e-6)
        assert np.array_equal(h1[0], h[t]) and np.array_equal(al1[0], al[t])


def pin_head_coordinates_do_not_route(orc):
    """[Explainer] worked example and [Paper] §3.3: only the last r coordinates are the key;
    coordinates outside the slice change the output but never the weights."""
    rng = _rng(3)
    d, r = 16, 5
    srcs = _rand_sources(rng, 4, 9, d)
    q = rng.standard_normal(r)
    h, al = orc.forward(srcs, q, r, 1e-6)
    moved = [s.copy() for s in srcs]
    for s in moved:
        s[:, : d - r] = rng.standard_normal((9, d - r)) * 10
    h2, al2 = orc.forward(moved, q, r, 1e-6)
    assert np.array_equal(al, al2)
    assert not np.allclose(h, h2)
    # and a change inside the slice does move the weights
    tail = [s.copy() for s in srcs]
    tail[0][:, d - 1] += 3.0
    _, al3 = orc.forward(tail, q, r, 1e-6)
    assert not np.allclose(al, al3)


def pin_slice_is_last_r(orc):
    """[Paper] §3.3: k = tail_r(o), the last r coordinates. A source whose only non-zero slice
    coordinate is d-1 scores q[r-1] * sqrt(r) at eps = 0 (its RMS is 1/sqrt r)."""
    d, r = 10, 4
    o = np.zeros((1, d))
    o[0, d - 1] = 1.0
    o[0, 0] = 5.0  # head coordinate, outside the key
    q = np.array([0.1, -0.2, 0.3, 0.7])
    z, rho = orc.scores([o], q, r, 0.0)
    assert abs(rho[0, 0] - 1 / math.sqrt(r)) < 1e-15
    assert abs(z[0, 0] - q[-1] * math.sqrt(r)) < 1e-14


def pin_r_equals_d_is_standard_attnres(orc):
    """[Explainer] and [Paper] §3.3: with r = d the read is standard AttnRes (full-width key,
    full-width RMSNorm). Compared with a separately written standard routine."""
    rng = _rng(4)
    for d in (1, 3, 16):
        srcs = _rand_sources(rng, 5, 11, d)
        q = rng.standard_normal(d)
        h, al = orc.forward(srcs, q, d, 1e-6)
        h2, al2 = orc.attnres_standard(srcs, q, 1e-6)
        assert np.allclose(al, al2, rtol=0, atol=1e-15)
        assert np.allclose(h, h2, rtol=1e-14, atol=1e-14)


def pin_scale_invariance(orc):
    """At eps = 0 the normalised key of c*o equals that of o for c > 0, so scaling one
    source's slice does not change its score."""
    rng = _rng(5)
    srcs = _rand_sources(rng, 3, 6, 9)
    q = rng.standard_normal(4)
    z, _ = orc.scores(srcs, q, 4, 0.0)
    z2, _ = orc.scores([srcs[0] * 37.5, srcs[1] * 0.01, srcs[2]], q, 4, 0.0)
    assert np.allclose(z, z2, rtol=1e-13, atol=1e-13)


def pin_permutation_equivariance(orc):
    """The read is a function of the set of sources: permuting them permutes the weights and
    leaves the output unchanged."""
    rng = _rng(6)
    srcs = _rand_sources(rng, 7, 5, 10)
    q = rng.standard_normal(3)
    h, al = orc.forward(srcs, q, 3, 1e-6)
    perm = [3, 0, 6, 2, 5, 1, 4]
    h2, al2 = orc.forward([srcs[p] for p in perm], q, 3, 1e-6)
    assert np.allclose(al2, al[:, perm], rtol=0, atol=1e-15)
    assert np.allclose(h2, h, rtol=1e-13, atol=1e-13)


def pin_single_source_identity(orc):
    """[Explainer] code comment and [Paper] App. E: the embedding-only read is the identity."""
    rng = _rng(7)
    o = rng.standard_normal((4, 6))
    h, al = orc.forward([o], rng.standard_normal(2), 2, 1e-6)
    assert np.array_equal(h, o) and np.array_equal(al, np.ones((4, 1)))


def pin_score_bound(orc):
    """|z_i| <= ||q||_2 sqrt(r): the normalised key has squared norm r*mu/(mu+eps) < r
    (Cauchy-Schwarz)."""
    rng = _rng(8)
    srcs = _rand_sources(rng, 6, 50, 12)
    q = rng.standard_normal(12)
    for r in (1, 5, 12):
        z, _ = orc.scores(srcs, q[:r], r, 1e-3)
        bound = np.linalg.norm(q[:r]) * math.sqrt(r)
        assert np.all(np.abs(z) < bound)


def pin_two_sources_logistic(orc):
    """With two sources the softmax is the logistic function of the score difference:
    alpha_1 / alpha_2 = exp(z_1 - z_2) (a textbook identity, checked through the scores the
    oracle reports)."""
    rng = _rng(9)
    srcs = _rand_sources(rng, 2, 20, 8)
    q = rng.standard_normal(3) * 3
    z, _ = orc.scores(srcs, q, 3, 1e-6)
    _, al = orc.forward(srcs, q, 3, 1e-6)
    assert np.allclose(np.log(al[:, 0] / al[:, 1]), z[:, 0] - z[:, 1], rtol=1e-12, atol=1e-12)


# --- a6-a7: two-phase statistics and merge ------------------------------------------------

def pin_stats_normalise_to_forward(orc):
    """[AttnRes-TR] Method and [Paper] §3.4: Phase-1 statistics over a source group, once
    normalised (acc / l), are that group's read; m is the largest score and l >= 1."""
    rng = _rng(10)
    srcs = _rand_sources(rng, 5, 13, 10)
    qs = rng.standard_normal((3, 4))
    m, l, acc = orc.stats(srcs, qs, 4, 1e-6)
    for s in range(3):
        h, _ = orc.forward(srcs, qs[s], 4, 1e-6)
        z, _ = orc.scores(srcs, qs[s], 4, 1e-6)
        assert np.allclose(acc[s] / l[s][:, None], h, rtol=1e-13, atol=1e-13)
        assert np.array_equal(m[s], z.max(axis=1))
        assert np.all(l[s] >= 1.0) and np.all(l[s] <= 5.0)


def pin_merge_equals_forward_on_union(orc):
    """[Paper] §3.4 and [Explainer] 'The contribution...': separately computed source groups
    merge by an online-softmax update. merge(stats(A), B) must equal forward(A u B) for every
    split of the sources, including an empty B."""
    rng = _rng(11)
    srcs = _rand_sources(rng, 6, 9, 14)
    q = rng.standard_normal(6)
    h_all, _ = orc.forward(srcs, q, 6, 1e-6)
    for k in range(1, 7):
        m, l, acc = orc.stats(srcs[:k], q[None, :], 6, 1e-6)
        h, m2, l2 = orc.merge(m[0], l[0], acc[0], srcs[k:], q, 6, 1e-6)
        assert np.allclose(h, h_all, rtol=1e-13, atol=1e-13), k
        m_all, l_all, _ = orc.stats(srcs, q[None, :], 6, 1e-6)
        assert np.allclose(m2, m_all[0], rtol=0, atol=1e-14)
        assert np.allclose(l2, l_all[0], rtol=1e-13, atol=0)


# --- a8: backward ------------------------------------------------------------------------

def _loss(orc, srcs, q, g, r, eps, fwd="forward"):
    h, _ = getattr(orc, fwd)(srcs, q, r, eps)
    return float(np.sum(h * g))


def pin_backward_finite_differences(orc):
    """The analytic backward ([Paper] App. B.3 Lemma 2, Cor. 2.1) against central differences
    of L = sum(g * h) with respect to every source coordinate and every query coordinate."""
    rng = _rng(12)
    T, d, r, n, eps = 3, 7, 3, 3, 1e-3
    srcs = _rand_sources(rng, n, T, d)
    q = rng.standard_normal(r)
    g = rng.standard_normal((T, d))
    dsrc, dq = orc.backward(srcs, q, g, r, eps)
    step = 1e-6
    for i in range(n):
        for t in range(T):
            for j in range(d):
                p = [s.copy() for s in srcs]
                p[i][t, j] += step
                lp = _loss(orc, p, q, g, r, eps)
                p[i][t, j] -= 2 * step
                lm = _loss(orc, p, q, g, r, eps)
                fd = (lp - lm) / (2 * step)
                assert abs(fd - dsrc[i][t, j]) < 1e-7 * max(1.0, abs(fd)), (i, t, j, fd,
                                                                            dsrc[i][t, j])
    for j in range(r):
        qp = q.copy()
        qp[j] += step
        lp = _loss(orc, srcs, qp, g, r, eps)
        qp[j] -= 2 * step
        lm = _loss(orc, srcs, qp, g, r, eps)
        fd = (lp - lm) / (2 * step)
        assert abs(fd - dq[j]) < 1e-7 * max(1.0, abs(fd)), (j, fd, dq[j])


def pin_backward_head_is_direct_gradient(orc):
    """[Paper] App. B.3 and [Explainer] 'What changes during learning': with slice
    normalisation the routing feedback lies only in the selected coordinates; elsewhere the
    source gradient is exactly alpha_i * g."""
    rng = _rng(13)
    T, d, r, n = 4, 11, 4, 5
    srcs = _rand_sources(rng, n, T, d)
    q = rng.standard_normal(r)
    g = rng.standard_normal((T, d))
    dsrc, _ = orc.backward(srcs, q, g, r, 1e-6)
    _, al = orc.forward(srcs, q, r, 1e-6)
    for i in range(n):
        assert np.array_equal(dsrc[i][:, : d - r], al[:, i:i + 1] * g[:, : d - r])
        assert not np.allclose(dsrc[i][:, d - r:], al[:, i:i + 1] * g[:, d - r:])


def pin_backward_jacobian_rank(orc):
    """[Paper] App. B.3 Cor. 2.3: the local value Jacobian dh/do_i has rank >= d - 1.
    Rows of the Jacobian are read off the backward with unit upstream gradients."""
    rng = _rng(14)
    T, d, r, n = 1, 6, 3, 3
    srcs = _rand_sources(rng, n, T, d)
    q = rng.standard_normal(r) * 2
    for i in range(n):
        J = np.zeros((d, d))
        for k in range(d):
            g = np.zeros((T, d))
            g[0, k] = 1.0
            dsrc, _ = orc.backward(srcs, q, g, r, 1e-6)
            J[k] = dsrc[i][0]
        assert np.linalg.matrix_rank(J) >= d - 1


def pin_backward_lemma2_sum(orc):
    """[Paper] App. B.3 Lemma 2: dh = sum_i alpha_i (o_i - h) dz_i, so the score gradients of
    one token sum to zero (the weights sum to one whatever the scores are)."""
    rng = _rng(15)
    T, d, r, n = 5, 9, 9, 4
    srcs = _rand_sources(rng, n, T, d)
    q = rng.standard_normal(r)
    g = rng.standard_normal((T, d))
    # dL/dq = sum_i dz_i kbar_i; with one query coordinate set to move all keys equally the
    # total must vanish: use constant keys in the slice so kbar_i is the same for every i.
    same = [s.copy() for s in srcs]
    for s in same:
        s[:, d - r:] = srcs[0][:, d - r:]
    _, dq = orc.backward(same, q, g, r, 1e-6)
    assert np.allclose(dq, 0.0, atol=1e-12)


def pin_fullrms_backward_finite_differences(orc):
    """Full-width-RMS control ([Paper] App. B.3 Cor. 2.2) against central differences."""
    rng = _rng(16)
    T, d, r, n, eps = 2, 6, 2, 3, 1e-3
    srcs = _rand_sources(rng, n, T, d)
    q = rng.standard_normal(r)
    g = rng.standard_normal((T, d))
    dsrc, dq = orc.backward_fullrms(srcs, q, g, r, eps)
    step = 1e-6
    for i in range(n):
        for t in range(T):
            for j in range(d):
                p = [s.copy() for s in srcs]
                p[i][t, j] += step
                lp = _loss(orc, p, q, g, r, eps, "forward_fullrms")
                p[i][t, j] -= 2 * step
                lm = _loss(orc, p, q, g, r, eps, "forward_fullrms")
                fd = (lp - lm) / (2 * step)
                assert abs(fd - dsrc[i][t, j]) < 1e-7 * max(1.0, abs(fd))
    for j in range(r):
        qp = q.copy()
        qp[j] += step
        lp = _loss(orc, srcs, qp, g, r, eps, "forward_fullrms")
        qp[j] -= 2 * step
        lm = _loss(orc, srcs, qp, g, r, eps, "forward_fullrms")
        assert abs((lp - lm) / (2 * step) - dq[j]) < 1e-7 * max(1.0, abs(dq[j]))


def pin_fullrms_at_r_equals_d(orc):
    """[Paper] §4.4 Eq. 13: at r = d slicing and full-width normalisation coincide."""
    rng = _rng(17)
    srcs = _rand_sources(rng, 4, 8, 10)
    q = rng.standard_normal(10)
    h, al = orc.forward_fullrms(srcs, q, 10, 1e-6)
    h2, al2 = orc.attnres_standard(srcs, q, 1e-6)
    assert np.allclose(al, al2, rtol=0, atol=1e-15) and np.allclose(h, h2, rtol=1e-14,
                                                                     atol=1e-14)


def pin_round_to_format(orc):
    """The storage rounding (IEEE round to nearest, ties to even) against library conversions:
    numpy's float32 cast for 24 bits and torch's bfloat16 cast for 8 bits, on random values,
    exact ties and values near 2^-126; plus hand-checked bfloat16 ties (1 + 2^-8 lies halfway
    between 1 and 1 + 2^-7 and goes to the even 1; 1 + 3 * 2^-8 goes up to 1 + 2^-6)."""
    import torch
    rng = _rng(30)
    x = np.concatenate([rng.standard_normal(4000) * 10.0 ** rng.integers(-6, 6, 4000),
                        1.0 + np.arange(-64, 64) * 2.0 ** -9, 1.0 + np.arange(-64, 64) * 2.0 ** -25,
                        rng.standard_normal(200) * 2.0 ** -126, [0.0, -0.0, 2.0 ** -130]])
    y24 = orc.round_to_format(x, 24)
    assert np.array_equal(y24, x.astype(np.float32).astype(np.float64))
    y8 = orc.round_to_format(x, 8)
    ref8 = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(y8, ref8)
    assert orc.round_to_format(np.array([1.0 + 2.0 ** -8]), 8)[0] == 1.0
    assert orc.round_to_format(np.array([1.0 + 3 * 2.0 ** -8]), 8)[0] == 1.0 + 2.0 ** -6
    normal = x[(np.abs(x) >= 2.0 ** -126) | (x == 0)]
    assert np.array_equal(orc.round_to_format(normal, 53), normal)


def pin_merge_accumulate_is_merge_of_updated_sum(orc):
    """The fused Phase-2 update ([Paper] §3.3 'Partial-block routing'): the site merges its
    statistics with b' = round(b + o), and with no earlier partial sum b' = o."""
    rng = _rng(31)
    T, d, r = 6, 16, 4
    A = _rand_sources(rng, 3, T, d)
    b = rng.standard_normal((T, d))
    o = rng.standard_normal((T, d))
    q = rng.standard_normal(r)
    m, l, acc = orc.stats(A, q[None, :], r, 1e-6)
    h, b2, m2, l2 = orc.merge_accumulate(m[0], l[0], acc[0], b, o, q, r, 1e-6, 8)
    bref = orc.round_to_format(b + o, 8)
    assert np.array_equal(b2, bref)
    href, mref, lref = orc.merge(m[0], l[0], acc[0], [bref], q, r, 1e-6)
    assert np.array_equal(h, href) and np.array_equal(m2, mref) and np.array_equal(l2, lref)
    h0, b0, _, _ = orc.merge_accumulate(m[0], l[0], acc[0], None, o, q, r, 1e-6, 53)
    assert np.array_equal(b0, o)
    h0ref, _, _ = orc.merge(m[0], l[0], acc[0], [o], q, r, 1e-6)
    assert np.array_equal(h0, h0ref)


def pin_merge_accumulate_block_equals_forward(orc):
    """A whole block by the two-phase schedule: Phase 1 over the completed sources A, then a
    site after two writes o1, o2 of the current block (b = o1 + o2, unrounded at 53 bits)
    reads exactly what one forward read over A and the sum o1 + o2 returns."""
    rng = _rng(32)
    T, d, r = 5, 12, 3
    A = _rand_sources(rng, 4, T, d)
    o1 = rng.standard_normal((T, d))
    o2 = rng.standard_normal((T, d)) * 2.0
    q = rng.standard_normal(r)
    m, l, acc = orc.stats(A, q[None, :], r, 1e-6)
    h, b, _, _ = orc.merge_accumulate(m[0], l[0], acc[0], o1, o2, q, r, 1e-6, 53)
    href, _ = orc.forward(A + [o1 + o2], q, r, 1e-6)
    assert np.allclose(h, href, rtol=1e-13, atol=1e-13)
    assert np.allclose(b, o1 + o2, rtol=0, atol=0)


def pin_fullrms_closed_form(orc):
    """[Paper] §4.4 Eq. 13 (control): the key is P_r o / sqrt(||o||^2 / d + eps), so the head
    coordinates enter through the denominator. At eps = 0, o_A = (1, 1, 1, 1) has full RMS 1
    and normalised key (1, 1); o_B = (2, 0, 0, 0) has full RMS 1 and key (0, 0). With
    q = (ln 3, 0) the scores are ln 3 and 0: weights (3/4, 1/4), h = (5/4, 3/4, 3/4, 3/4).
    Moving o_A's head to (3, 1) makes its full RMS sqrt 3, so its score is ln 3 / sqrt 3."""
    q = np.array([math.log(3.0), 0.0])
    oA = np.array([[1.0, 1.0, 1.0, 1.0]])
    oB = np.array([[2.0, 0.0, 0.0, 0.0]])
    h, al = orc.forward_fullrms([oA, oB], q, 2, 0.0)
    assert np.allclose(al[0], [0.75, 0.25], rtol=0, atol=1e-15), al
    assert np.allclose(h[0], [1.25, 0.75, 0.75, 0.75], rtol=0, atol=1e-15), h
    oA2 = np.array([[3.0, 1.0, 1.0, 1.0]])
    _, al2 = orc.forward_fullrms([oA2, oB], q, 2, 0.0)
    e = math.exp(math.log(3.0) / math.sqrt(3.0))
    assert np.allclose(al2[0], [e / (e + 1.0), 1.0 / (e + 1.0)], rtol=0, atol=1e-15), al2
    # eps is added to the mean of squares: eps = 3 makes o_A's RMS 2 and its score ln 3 / 2
    _, al3 = orc.forward_fullrms([oA, oB], q, 2, 3.0)
    zB = 0.0
    zA = math.log(3.0) / 2.0
    wA = math.exp(zA) / (math.exp(zA) + math.exp(zB))
    assert abs(al3[0, 0] - wA) < 1e-15, al3


def _worked_keys():
    """The worked example's keys (1, 0) and (0, 1) as separate key rows."""
    return np.array([[1.0, 0.0]]), np.array([[0.0, 1.0]])


def pin_keys_worked_example(orc):
    """Separate-key read ([Paper] App. C.1: each source's key is its own r-wide vector,
    RMS-normalised). With the worked example's keys (1, 0) and (0, 1) held apart from the
    values and q = (ln 3 / sqrt 2, 0), the weights are (3/4, 1/4) whatever the values hold,
    their last coordinates included, and h = 3/4 o_A + 1/4 o_B."""
    q = np.array([math.log(3.0) / math.sqrt(2.0), 0.0])
    kA, kB = _worked_keys()
    oA = np.array([[4.0, -1.0, 7.0, -2.0, 0.5]])
    oB = np.array([[0.0, 3.0, 5.0, 3.0, -8.0]])
    h, al = orc.forward_keys([oA, oB], [kA, kB], q, 2, 0.0)
    assert np.allclose(al[0], [0.75, 0.25], rtol=0, atol=1e-15), al
    assert np.allclose(h[0], 0.75 * oA[0] + 0.25 * oB[0], rtol=0, atol=1e-14), h


def pin_keys_equal_tail_is_slice_read(orc):
    """When each source's key is a copy of its own last r coordinates the separate-key read is
    the sliced read ([Paper] §3.3 vs App. C.1). The keys sit in wider arrays (row stride > r),
    so the key stride is exercised too."""
    rng = _rng(18)
    T, d, r, n = 5, 12, 4, 3
    srcs = _rand_sources(rng, n, T, d)
    keys = []
    for s in srcs:
        k = rng.standard_normal((T, r + 3))
        k[:, :r] = s[:, d - r:]
        keys.append(k)
    q = rng.standard_normal(r)
    h, al = orc.forward_keys(srcs, keys, q, r, 1e-6)
    h2, al2 = orc.forward(srcs, q, r, 1e-6)
    assert np.allclose(al, al2, rtol=0, atol=1e-15) and np.allclose(h, h2, rtol=1e-14,
                                                                     atol=1e-14)


def pin_keys_values_do_not_route(orc):
    """With separate keys the values only carry content: changing every value leaves the
    weights unchanged, and h is linear in the values."""
    rng = _rng(19)
    T, d, r, n = 4, 6, 3, 4
    srcs = _rand_sources(rng, n, T, d)
    other = _rand_sources(rng, n, T, d)
    keys = _rand_sources(rng, n, T, r)
    q = rng.standard_normal(r)
    h1, al1 = orc.forward_keys(srcs, keys, q, r, 1e-6)
    h2, al2 = orc.forward_keys(other, keys, q, r, 1e-6)
    assert np.array_equal(al1, al2)
    both = [a + b for a, b in zip(srcs, other)]
    h3, _ = orc.forward_keys(both, keys, q, r, 1e-6)
    assert np.allclose(h3, h1 + h2, rtol=1e-13, atol=1e-13)


def pin_nan_on_zero_slice(orc):
    """[Explainer]: eps > 0 prevents division by zero. At eps = 0 an all-zero slice gives 0/0,
    and the read returns NaN for that token rather than a made-up value."""
    o = np.zeros((1, 4))
    o2 = np.ones((1, 4))
    h, al = orc.forward([o, o2], np.array([1.0, 1.0]), 2, 0.0)
    assert np.all(np.isnan(al)) and np.all(np.isnan(h))
    h, al = orc.forward([o, o2], np.array([1.0, 1.0]), 2, 1e-6)
    assert np.all(np.isfinite(h))


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
