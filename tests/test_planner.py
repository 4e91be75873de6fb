"""Checkpoint placement: oracle pins, then the library's host planner against
the oracle.  CPU only (the planner does no device work).

Source: "Sparse prefix caching for hybrid and recurrent LLM serving" (arXiv
2605.05219), §3 (objective R), §4 (Theorem 1, Theorem 2, Lemma 1, and the
plug-in and drift guarantees of Theorems 3 and 4) and §5 (the uniform-spacing
baseline: gaps that differ by at most one).
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


def _empirical(rng, p, T):
    """Normalised histogram of T i.i.d. draws of d ~ p on 0..N."""
    return np.bincount(rng.choice(len(p), size=T, p=p), minlength=len(p)) / T


def test_theorem3_plugin_guarantee():
    """A placement optimal for the empirical distribution p^ of T requests costs,
    under the true p, at most V(p, M) + 2 N TV(p^, p)."""
    rng = np.random.default_rng(7)
    for _ in range(40):
        N = int(rng.integers(2, 40))
        M = int(rng.integers(1, min(N, 6) + 1))
        p = rng.random(N + 1) ** 3; p /= p.sum()
        ph = _empirical(rng, p, int(rng.integers(5, 200)))
        tv = 0.5 * np.abs(p - ph).sum()
        _, g_hat = OP.dp_optimum(ph, M)
        v, _ = OP.dp_optimum(p, M)
        r = OP.expected_recompute(p, g_hat)
        assert v - 1e-12 <= r <= v + 2 * N * tv + 1e-12


def test_theorem4_drift_guarantee():
    """Placements recomputed from a sliding window of drifting requests: under the
    next step's distribution p_T they cost at most V(p_T, M) + 2 N eps, with
    eps = TV(p_T, window average)."""
    rng = np.random.default_rng(8)
    N, M, W = 60, 4, 25
    a = rng.random(N + 1); a /= a.sum()
    b = rng.random(N + 1) ** 4; b /= b.sum()
    steps = 120
    dists = [(1 - t / steps) * a + (t / steps) * b for t in range(steps + 1)]
    draws = [rng.choice(N + 1, p=d) for d in dists[:-1]]
    for T in range(W, steps, 7):
        window = np.bincount(draws[T - W:T], minlength=N + 1) / W
        p_next = dists[T]
        eps = 0.5 * np.abs(p_next - window).sum()
        _, g_hat = OP.dp_optimum(window, M)
        v, _ = OP.dp_optimum(p_next, M)
        assert OP.expected_recompute(p_next, g_hat) <= v + 2 * N * eps + 1e-12


# ---- the library's planner against the oracle --------------------------------

@pytest.fixture(scope="module")
def gdn():
    import gated_delta_rule_scan_amd as g
    g.load()
    return g


def _families(rng, N):
    yield "uniform", _uniform(N)
    yield "random", rng.random(N + 1)
    sparse = rng.random(N + 1) * (rng.random(N + 1) < 0.2)
    yield "sparse", sparse
    yield "geometric", 0.97 ** np.arange(N + 1)
    yield "spikes", np.bincount(rng.integers(0, N + 1, 5), minlength=N + 1).astype(float)
    yield "zero", np.zeros(N + 1)


def test_lib_expected_recompute_matches_oracle(gdn):
    rng = np.random.default_rng(6)
    for _ in range(100):
        N = int(rng.integers(0, 80))
        M = int(rng.integers(0, N + 1))
        p = rng.random(N + 1)
        pos = sorted(rng.choice(np.arange(1, N + 1), M, replace=False).tolist()) if M else []
        assert gdn.expected_recompute(p, pos) == pytest.approx(OP.expected_recompute(p, pos), rel=1e-12, abs=1e-12)
    # invalid placements and weights are rejected
    assert gdn.expected_recompute([0.1, 0.2, 0.3], [2, 2]) == -1.0
    assert gdn.expected_recompute([0.1, 0.2, 0.3], [3]) == -1.0
    assert gdn.expected_recompute([0.1, -0.2, 0.3], [1]) == -1.0
    assert gdn.expected_recompute([0.1, float("nan"), 0.3], [1]) == -1.0


def test_lib_balanced_is_theorem1_placement(gdn):
    for N, M in [(1, 1), (2, 1), (10, 3), (8192, 8), (32768, 16), (65536, 16), (100, 100)]:
        pos = gdn.balanced_checkpoints(N, M).tolist()
        assert pos == OP.gaps_to_positions(OP.balanced_gaps(N, M))
        g = OP.positions_to_gaps(pos, N)
        assert sum(g) == N + 1 and min(g) >= 1 and max(g) - min(g) <= 1
    with pytest.raises(Exception):
        gdn.balanced_checkpoints(3, 4)


@pytest.mark.parametrize("N", [1, 2, 7, 40, 150])
def test_lib_plan_matches_dp_oracle(gdn, N):
    rng = np.random.default_rng(100 + N)
    for M in sorted({0, 1, 2, 3, 5, 8, N} & set(range(N + 1))):
        for name, p in _families(rng, N):
            pos, cost = gdn.plan_checkpoints(p, M)
            want, _ = OP.dp_optimum(p, M)
            scale = max(1.0, float(np.sum(p)) * N)
            assert cost == pytest.approx(want, rel=1e-9, abs=1e-12 * scale), (name, N, M)
            pos = pos.tolist()
            assert len(pos) == M and all(1 <= x <= N for x in pos) and pos == sorted(set(pos))
            # the returned placement reaches the minimum
            assert OP.expected_recompute(p, pos) == pytest.approx(want, rel=1e-9, abs=1e-12 * scale)


def test_lib_plan_from_samples_keeps_the_plugin_bound(gdn):
    """The library's plan built from an empirical distribution obeys Theorem 3
    under the true distribution (the library's plan and the oracle's optimum may
    differ among ties, the bound may not)."""
    rng = np.random.default_rng(9)
    for _ in range(25):
        N = int(rng.integers(5, 300))
        M = int(rng.integers(1, min(N, 16) + 1))
        p = rng.random(N + 1) ** 2; p /= p.sum()
        ph = _empirical(rng, p, 400)
        tv = 0.5 * np.abs(p - ph).sum()
        pos, _ = gdn.plan_checkpoints(ph, M)
        v, _ = OP.dp_optimum(p, M)
        assert OP.expected_recompute(p, pos.tolist()) <= v + 2 * N * tv + 1e-9


def test_lib_plan_is_a_brute_force_optimum(gdn):
    rng = np.random.default_rng(7)
    for _ in range(80):
        N = int(rng.integers(1, 10))
        M = int(rng.integers(0, min(N, 4) + 1))
        p = rng.random(N + 1) * (rng.random(N + 1) < 0.6)
        best, argmins = OP.brute_force_optimum(p, M, rel_tol=1e-9)
        pos, cost = gdn.plan_checkpoints(p, M)
        assert cost == pytest.approx(best, rel=1e-9, abs=1e-12)
        assert tuple(pos.tolist()) in argmins


def _recompute_vec(p, pos):
    """R by the definition, vectorised over depths (test helper)."""
    N = len(p) - 1
    d = np.arange(N + 1)
    c = np.r_[0, np.asarray(pos, dtype=np.int64)]
    last = c[np.searchsorted(c, d, side="right") - 1]
    return float(np.dot(p, d - last))


def test_lib_plan_large_sizes(gdn):
    """N = 65536, M = 16 (the prefill-with-emission shape): the plan's cost is
    what its positions give, no single checkpoint moved by one position does
    better, it beats the balanced and random placements, and for uniform p it
    ties the balanced placement (Theorem 1)."""
    rng = np.random.default_rng(8)
    N, M = 65536, 16
    x = np.arange(N + 1) / N
    p = np.exp(-((x - 0.3) / 0.05) ** 2) + 0.5 * np.exp(-((x - 0.8) / 0.02) ** 2) + 0.05
    p[0] = 0.1
    p /= p.sum()
    t0 = time.perf_counter()
    pos, cost = gdn.plan_checkpoints(p, M)
    dt = time.perf_counter() - t0
    assert dt < 5.0, dt
    pos = pos.tolist()
    assert cost == pytest.approx(_recompute_vec(p, pos), rel=1e-9)
    for i in range(M):
        for step in (-1, 1):
            q = list(pos)
            q[i] += step
            if (i > 0 and q[i] <= q[i - 1]) or (i + 1 < M and q[i] >= q[i + 1]) or not (1 <= q[i] <= N):
                continue
            assert _recompute_vec(p, q) >= cost - 1e-9 * cost
    bal = gdn.balanced_checkpoints(N, M)
    assert cost <= _recompute_vec(p, bal) + 1e-12
    for _ in range(5):
        rnd = np.sort(rng.choice(np.arange(1, N + 1), M, replace=False))
        assert cost <= _recompute_vec(p, rnd) + 1e-12
    pu = _uniform(N)
    posu, costu = gdn.plan_checkpoints(pu, M)
    assert costu == pytest.approx(_recompute_vec(pu, bal), rel=1e-9)
    g = OP.positions_to_gaps(posu.tolist(), N)
    assert max(g) - min(g) <= 1


def test_lib_plan_edge_cases_and_errors(gdn):
    p = np.r_[0.0, np.ones(10)]
    pos, cost = gdn.plan_checkpoints(p, 0)
    assert pos.size == 0 and cost == pytest.approx(sum(range(11)))
    pos, cost = gdn.plan_checkpoints(p, 10)
    assert pos.tolist() == list(range(1, 11)) and cost == 0.0
    pos, cost = gdn.plan_checkpoints(np.zeros(11), 3)
    assert cost == 0.0 and pos.tolist() == sorted(set(pos.tolist()))
    for bad_p, M in [([1.0], 0), (p, 11), (p, -1), (np.r_[p[:-1], -1.0], 2), (np.r_[p[:-1], np.inf], 2)]:
        with pytest.raises(gdn.GDNError) as e:
            gdn.plan_checkpoints(bad_p, M)
        assert e.value.status == 1
