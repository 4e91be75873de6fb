"""Checkpoint placement: oracle pins, then the library's host planner against
the oracle.  CPU only (the planner does no device work).

Source: "Sparse prefix caching for hybrid and recurrent LLM serving" (arXiv
2605.05219), §3 (objective R), §4 (Theorem 1, Theorem 2, Lemma 1) and §5
(the uniform-spacing baseline: gaps that differ by at most one).
"""
import itertools
import time

import numpy as np
import pytest

from oracle import planner as OP


# ---- oracle pins -------------------------------------------------------------

def _uniform(N):
    return np.r_[0.0, np.full(N, 1.0 / N)]


def test_recompute_closed_form_uniform():
    """p uniform on 1..N: each gap g contributes 0 + 1 + ... + (g - 1) = g (g-1)/2
    recomputed tokens (the quantity phi(g) in the proof of Theorem 1), so
    R = sum g_i (g_i - 1) / (2 N)."""
    rng = np.random.default_rng(1)
    for _ in range(200):
        N = int(rng.integers(1, 60))
        M = int(rng.integers(0, N + 1))
        pos = sorted(rng.choice(np.arange(1, N + 1), M, replace=False).tolist())
        g = OP.positions_to_gaps(pos, N)
        assert sum(g) == N + 1 and min(g) >= 1
        assert OP.gaps_to_positions(g) == pos
        want = sum(x * (x - 1) for x in g) / (2.0 * N)
        assert OP.expected_recompute(_uniform(N), pos) == pytest.approx(want, rel=1e-12, abs=1e-15)


def test_recompute_special_cases():
    rng = np.random.default_rng(2)
    p = rng.random(21)
    N = 20
    # no checkpoint: every depth recomputes from the zero state
    assert OP.expected_recompute(p, []) == pytest.approx(sum(d * p[d] for d in range(N + 1)))
    # a checkpoint at every position: nothing to recompute
    assert OP.expected_recompute(p, list(range(1, N + 1))) == 0.0
    # a depth equal to a checkpoint recomputes nothing; one past it, one token
    assert OP.recompute_len([5, 9], 9) == 0 and OP.recompute_len([5, 9], 10) == 1
    assert OP.recompute_len([5, 9], 4) == 4 and OP.recompute_len([5, 9], 0) == 0


def test_theorem1_exchange_identity():
    """Proof of Theorem 1: moving one token from gap i to gap j changes N R by
    phi(g_i) + phi(g_j) - phi(g_i - 1) - phi(g_j + 1) = g_i - g_j - 1."""
    rng = np.random.default_rng(3)
    for _ in range(200):
        N = int(rng.integers(4, 50))
        M = int(rng.integers(1, min(N, 8) + 1))
        pos = sorted(rng.choice(np.arange(1, N + 1), M, replace=False).tolist())
        g = OP.positions_to_gaps(pos, N)
        i, j = rng.choice(len(g), 2, replace=False)
        if g[i] < 2:
            continue
        g2 = list(g)
        g2[i] -= 1
        g2[j] += 1
        p = _uniform(N)
        diff = N * (OP.expected_recompute(p, pos) - OP.expected_recompute(p, OP.gaps_to_positions(g2)))
        assert diff == pytest.approx(g[i] - g[j] - 1, abs=1e-9)


def test_theorem1_by_brute_force():
    """p uniform on 1..N: every optimal placement has gaps that differ by at most
    one, and the balanced placement is optimal."""
    for N in range(2, 12):
        for M in range(1, min(N, 4) + 1):
            p = _uniform(N)
            best, argmins = OP.brute_force_optimum(p, M)
            for pos in argmins:
                g = OP.positions_to_gaps(pos, N)
                assert max(g) - min(g) <= 1, (N, M, pos)
            bal = OP.gaps_to_positions(OP.balanced_gaps(N, M))
            assert OP.expected_recompute(p, bal) == pytest.approx(best, rel=1e-12)


def test_dp_oracle_matches_brute_force():
    rng = np.random.default_rng(4)
    for _ in range(60):
        N = int(rng.integers(1, 10))
        M = int(rng.integers(0, min(N, 4) + 1))
        p = rng.random(N + 1) * (rng.random(N + 1) < 0.7)
        best, argmins = OP.brute_force_optimum(p, M)
        cost, pos = OP.dp_optimum(p, M)
        assert cost == pytest.approx(best, rel=1e-12, abs=1e-15)
        assert tuple(pos) in argmins


def test_lemma1_lipschitz():
    """|V(p, M) - V(q, M)| <= N TV(p, q) for distributions p, q on 0..N."""
    rng = np.random.default_rng(5)
    for _ in range(30):
        N = int(rng.integers(2, 30))
        M = int(rng.integers(1, min(N, 5) + 1))
        p = rng.random(N + 1); p /= p.sum()
        q = rng.random(N + 1); q /= q.sum()
        tv = 0.5 * np.abs(p - q).sum()
        vp, _ = OP.dp_optimum(p, M)
        vq, _ = OP.dp_optimum(q, M)
        assert abs(vp - vq) <= N * tv + 1e-12
