"""The oracle against the pages' facts and mathematical invariants (CPU only)."""
import numpy as np
import pytest

import oracle_pins
from oracle_pins import ALL_PINS


@pytest.mark.parametrize("pin", ALL_PINS, ids=[p.__name__ for p in ALL_PINS])
def test_pin(orc, pin):
    pin(orc)


def test_backward_fd_32_token_slice(orc):
    """Finite differences on a 32-token slice at the backward workload's width
    (d = 4096, r = 1024, 10 sources), on sampled coordinates: head and tail of every
    source and a spread of query coordinates."""
    rng = np.random.default_rng(20)
    T, d, r, n, eps = 32, 4096, 1024, 10, 1e-6
    srcs = [rng.standard_normal((T, d)) * rng.uniform(0.5, 4.0) for _ in range(n)]
    q = rng.standard_normal(r)
    g = rng.standard_normal((T, d))
    dsrc, dq = orc.backward(srcs, q, g, r, eps)

    def loss(ss, qq):
        h, _ = orc.forward(ss, qq, r, eps)
        return float(np.sum(h * g))

    step = 1e-5
    picks = [(i, int(rng.integers(T)), int(j)) for i in range(n)
             for j in (0, d // 2, d - r - 1, d - r, d - r + 7, d - 1)]
    for i, t, j in picks:
        # only token t depends on o_i[t, j]; perturb a one-row slice to keep this fast
        sl = [s[t:t + 1].copy() for s in srcs]
        gl = g[t:t + 1]
        sl[i][0, j] += step
        hp, _ = orc.forward(sl, q, r, eps)
        sl[i][0, j] -= 2 * step
        hm, _ = orc.forward(sl, q, r, eps)
        fd = float(np.sum((hp - hm) * gl)) / (2 * step)
        assert abs(fd - dsrc[i][t, j]) < 1e-6 * max(1.0, abs(fd)), (i, t, j, fd, dsrc[i][t, j])
    base = loss(srcs, q)
    assert np.isfinite(base)
    for j in (0, 1, r // 3, r // 2, r - 1):
        qp = q.copy()
        qp[j] += step
        lp = loss(srcs, qp)
        qp[j] -= 2 * step
        lm = loss(srcs, qp)
        fd = (lp - lm) / (2 * step)
        assert abs(fd - dq[j]) < 1e-6 * max(1.0, abs(fd)), (j, fd, dq[j])


def test_pins_module_lists_every_pin():
    names = [p.__name__ for p in ALL_PINS]
    assert len(names) == len(set(names)) >= 15
    assert all(callable(getattr(oracle_pins, n)) for n in names)


def test_block_schedule_golden():
    """The block-routing schedule against the explainer's six-write example (its entries after
    writes three and four; tests/golden/block_schedule_example.json), the block-end rule, full
    routing as N = M, and the production-width reading of 93 writes in 8 blocks."""
    import json
    import os

    import oracle

    with open(os.path.join(os.path.dirname(__file__), "golden",
                           "block_schedule_example.json")) as f:
        g = json.load(f)
    M, N = g["M"], g["N"]
    assert oracle.block_ends(M, N) == g["expected_ends"]
    for w, want in g["expected_sources_after_write"].items():
        assert oracle.block_sources(M, N, int(w)) == want, w
    # full routing (every write its own block): the read after write w sees w + 1 sources
    assert all(oracle.block_sources(48, 48, w) == [[i] for i in range(w + 1)] for w in range(49))
    # 93 writes in 8 blocks: blocks of 11-12 writes, at most N + 1 = 9 sources at any read
    assert oracle.block_ends(93, 8) == [12, 24, 35, 47, 59, 70, 82, 93]
    counts = [len(oracle.block_sources(93, 8, w)) for w in range(94)]
    assert max(counts) == 9 and counts[93] == 9 and counts[12] == 2
    # every write lands in exactly one source at every read
    for w in range(94):
        flat = sorted(i for s in oracle.block_sources(93, 8, w) for i in s)
        assert flat == list(range(w + 1))
