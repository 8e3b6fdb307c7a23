"""Tolerances for comparing the HIP path with the oracle.

The bars (element by element):
  * weights alpha: |alpha - alpha_ref| <= 1e-6;
  * fp32 output: |y - h_ref| <= 1e-5 * max|v| with v the source values of the read;
  * bf16 output: |y - h_ref| <= ulp_bf16(h_ref) + (n + 3 + 2k) * 2^-24 * sum_i alpha_i |o_ij|.
    The first term is one bf16 ulp of the value; the second bounds the float32 arithmetic
    before that rounding (it only matters under cancellation): n roundings of the n fused
    multiply-adds, one of each weight's float32 rounding, one of 1/l and one of the final
    scaling by it (the two-pass read has neither of the last two), and two for each of the k
    times the online fold moves its reference and rescales the accumulator (the scale factor's
    rounding and the product's). k is counted per row from the oracle's weights.
  * Phase-1 statistics: m within one float32 rounding; l and acc within the float32
    accumulation bound after rescaling the oracle to the kernel's m.
  * backward: dsrc_i within 1e-5 * max|dsrc_i ref| per source (plus one bf16 ulp of the
    value for bf16 gradients); dq within 1e-5 * sum_t sum_i |dz_ti| * max_j |kbar_tij|.
"""
from __future__ import annotations

import numpy as np

U = 2.0 ** -24


def ulp_bf16(x):
    ax = np.abs(np.asarray(x, dtype=np.float64))
    tiny = 2.0 ** -126
    e = np.floor(np.log2(np.maximum(ax, tiny)))
    return np.where(ax < tiny, 2.0 ** -133, 2.0 ** (e - 7))


def _report(err, tol, where):
    bad = ~(err <= tol)
    if bad.any():
        idx = np.unravel_index(np.argmax(np.where(bad, err / np.maximum(tol, 1e-300), 0)),
                               err.shape)
        raise AssertionError(f"{where}: {int(bad.sum())} of {err.size} elements out of "
                             f"tolerance; worst at {idx}: err {err[idx]:.3e} > tol {tol[idx]:.3e}")


def _nan_equal_mask(a, b):
    return np.isnan(a) & np.isnan(b)


LAZY_RESCALE = 8.0  # the online fold moves its reference when a score passes it by more


def lazy_rescales(alpha_ref):
    """Per row, how often an online-softmax fold over the sources in order rescales its
    accumulator after the first source: a score more than LAZY_RESCALE above the reference
    becomes the new reference. Score differences are read from the oracle's weights
    (z_i - z_j = ln(alpha_i / alpha_j)); a margin makes borderline rows count (more slack)."""
    with np.errstate(divide="ignore"):
        lz = np.log(np.asarray(alpha_ref, dtype=np.float64))
    k = np.zeros(lz.shape[0])
    ref = lz[:, 0].copy()
    for i in range(1, lz.shape[1]):
        grow = lz[:, i] > ref + LAZY_RESCALE - 1e-6
        k += grow
        ref = np.where(grow, lz[:, i], ref)
    return k


def assert_read(y64, h_ref, alpha_ref, srcs64, io, where="read"):
    """y64: kernel output decoded to float64 [T, d]; h_ref, alpha_ref from the oracle."""
    n = len(srcs64)
    if io == "bf16":
        mag = np.zeros_like(h_ref)
        for i in range(n):
            mag += alpha_ref[:, i:i + 1] * np.abs(srcs64[i])
        slack = (n + 3 + 2 * lazy_rescales(alpha_ref))[:, None]
        tol = ulp_bf16(h_ref) + slack * U * mag
    else:
        vmax = max(float(np.nanmax(np.abs(s))) for s in srcs64)
        tol = np.full_like(h_ref, 1e-5 * vmax)
    err = np.abs(y64 - h_ref)
    err[_nan_equal_mask(y64, h_ref)] = 0.0
    _report(err, tol, where)


def assert_weights(a64, a_ref, where="weights"):
    err = np.abs(a64 - a_ref)
    err[_nan_equal_mask(a64, a_ref)] = 0.0
    _report(err, np.full_like(err, 1e-6), where)


def assert_stats(m_g, l_g, acc_g, m_o, l_o, acc_o, z_o, srcs64, acc_io, where="stats"):
    """Kernel statistics against the oracle's, rescaled to the kernel's rounded maximum.
    m_*, l_* are [T]; acc_* are [T, d]; z_o [T, n] are the oracle's scores."""
    n = len(srcs64)
    _report(np.abs(m_g - m_o), 2.0 ** -23 * np.abs(m_o) + 1e-12, where + " m")
    s = np.exp(m_o - m_g)
    l_ref = l_o * s
    _report(np.abs(l_g - l_ref), 4 * U * l_ref, where + " l")
    acc_ref = acc_o * s[:, None]
    e = np.exp(z_o - m_g[:, None])
    mag = np.zeros_like(acc_ref)
    for i in range(n):
        mag += e[:, i:i + 1] * np.abs(srcs64[i])
    tol = (n + 3) * U * mag
    if acc_io == "bf16":
        tol = tol + ulp_bf16(acc_ref)
    _report(np.abs(acc_g - acc_ref), tol, where + " acc")


def assert_merge(y64, h_ref, w_prior, acc_norm, w_extra, extra64, io, where="merge"):
    """h = w_prior * (acc / l) + sum_b w_b o_b; w_* from the oracle (w_prior [T], w_extra
    [T, n_extra]); acc_norm = acc / l [T, d]. The slack counts, besides the read's terms, the
    stored accumulator's scaling, and one possible rescale per extra source (the fold starts
    from the Phase-1 maximum)."""
    mag = w_prior[:, None] * np.abs(acc_norm)
    for i, b in enumerate(extra64):
        mag += w_extra[:, i:i + 1] * np.abs(b)
    n = len(extra64) + 1
    slack = n + 4 + 2 * len(extra64)
    if io == "bf16":
        tol = ulp_bf16(h_ref) + slack * U * mag
    else:
        vmax = max([float(np.abs(acc_norm).max())] + [float(np.abs(b).max()) for b in extra64])
        tol = np.full_like(h_ref, 1e-5 * vmax) + slack * U * mag
    err = np.abs(y64 - h_ref)
    err[_nan_equal_mask(y64, h_ref)] = 0.0
    _report(err, tol, where)


def assert_dsrc(g64, g_ref, where="dsrc"):
    tol = np.full_like(g_ref, 1e-5 * max(float(np.abs(g_ref).max()), 1e-30))
    _report(np.abs(g64 - g_ref), tol, where)


def assert_dsrc_bf16(g64, g_ref, where="dsrc"):
    """bf16 source gradients: the float32 bar of assert_dsrc plus one bf16 ulp of the value
    (the kernel rounds its float32 result to nearest even once)."""
    tol = ulp_bf16(g_ref) + 1e-5 * max(float(np.abs(g_ref).max()), 1e-30)
    _report(np.abs(g64 - g_ref), tol, where)


def dq_bound(srcs64, q, dout64, alpha, h, r, eps):
    """The dq tolerance in units of the 1e-5 bar (assert_dq takes 1e-5 times this; sums over row
    chunks add): sum_t sum_i |dz_ti| max_j |kbar_tij|, plus 1e5 times the absolute error of
    dz_ti = alpha_ti (s_ti - sbar_t) that float64 leaves on either side, where the two sides sum
    s_ti = g_t . o_ti (d exact products) and sbar_t in different orders: at most
    alpha_ti (d + 2) 2^-53 (S_ti + sum_j alpha_tj S_tj) with S_ti = sum_c |g_tc o_tic|. That term
    only matters when the softmax saturates, where s_ti - sbar_t cancels to almost nothing and
    dq is rounding noise (LR-AttnRes paper, App. B.3, Lemma 2)."""
    d = srcs64[0].shape[1]
    total = 0.0
    gamma = (d + 2) * 2.0 ** -53
    big = [np.sum(np.abs(dout64 * o), axis=1) for o in srcs64]        # S_ti
    sbar_mag = sum(alpha[:, j] * big[j] for j in range(len(srcs64)))   # sum_j alpha_tj S_tj
    for i, o in enumerate(srcs64):
        dz = alpha[:, i] * np.sum(dout64 * (o - h), axis=1)
        k = o[:, d - r:]
        rho = np.sqrt(np.mean(k * k, axis=1) + eps)
        kmax = np.max(np.abs(k), axis=1) / rho
        cancel = alpha[:, i] * gamma * (big[i] + sbar_mag)
        total += float(np.sum((np.abs(dz) + 1e5 * cancel) * kmax))
    return total


def assert_dq(dq_g, dq_o, bound, where="dq"):
    _report(np.abs(dq_g - dq_o), np.full_like(dq_o, 1e-5 * bound + 1e-30), where)
