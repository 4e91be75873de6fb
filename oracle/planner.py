"""Checkpoint-placement oracle (fp64, plain loops).

TEST INFRASTRUCTURE ONLY, like the rest of ``oracle``: imported by ``tests/``
alone, never by the product path, and it imports nothing from it.

Source: "Sparse prefix caching for hybrid and recurrent LLM serving"
(arXiv 2605.05219, translated page), §3 (problem statement) and §4
(Theorems 1 and 2, Lemma 1).

§3: a cached prefix of N tokens keeps exact states at positions
1 <= c_1 < ... < c_M <= N, described by the gap vector g_1..g_K, K = M + 1,
each g_i >= 1 and sum g_i = N + 1, with c_i = g_1 + ... + g_i.  A request
that matches to depth d resumes from the deepest checkpoint at or before d
and recomputes f_g(d) = d - max{c_i : c_i <= d} tokens (c_0 = 0 when none
qualifies, which is how a garbled index of the page is read here); f_g(0) = 0.
The objective is R(p, g) = E_{d ~ p}[f_g(d)] over depths 0..N.

§4: Theorem 1 (p uniform on 1..N: every minimiser has gaps differing by at
most one), Theorem 2 (any p: a dynamic programme over prefixes and checkpoint
counts, DP[t][k] = min_{s<t} DP[s][k-1] + C(s+1, t)), Lemma 1
(|V(p, M) - V(q, M)| <= N TV(p, q), V the optimal value).

Functions here follow those statements directly: the objective is summed
depth by depth, the optimum is found by enumerating every gap vector (tiny
sizes) or by the page's recurrence with interval costs summed term by term.
Pins: ``tests/test_planner.py``.
"""
from __future__ import annotations

import itertools
from typing import List, Sequence, Tuple

import numpy as np

__all__ = [
    "gaps_to_positions",
    "positions_to_gaps",
    "recompute_len",
    "expected_recompute",
    "balanced_gaps",
    "brute_force_optimum",
    "dp_optimum",
]


def gaps_to_positions(g: Sequence[int]) -> List[int]:
    """c_i = g_1 + ... + g_i for i = 1..K-1 (the last gap ends at N + 1)."""
    out, s = [], 0
    for gi in g[:-1]:
        s += int(gi)
        out.append(s)
    return out


def positions_to_gaps(positions: Sequence[int], N: int) -> List[int]:
    c = [0] + [int(x) for x in positions] + [N + 1]
    return [c[i + 1] - c[i] for i in range(len(c) - 1)]


def recompute_len(positions: Sequence[int], d: int) -> int:
    """f_g(d) = d - (deepest checkpoint <= d, or 0), and 0 for d = 0 (§3)."""
    if d == 0:
        return 0
    best = 0
    for c in positions:
        if c <= d and c > best:
            best = c
    return d - best


def expected_recompute(p: Sequence[float], positions: Sequence[int]) -> float:
    """R = sum over depths d = 0..N of p(d) f_g(d), N = len(p) - 1 (§3)."""
    return float(sum(float(p[d]) * recompute_len(positions, d) for d in range(len(p))))


def balanced_gaps(N: int, M: int) -> List[int]:
    """A gap vector with K = M + 1 gaps of sizes q or q + 1, N + 1 = q K + rho
    (the construction in the proof of Theorem 1): here the rho larger gaps
    come last, which gives the positions floor(i (N + 1) / (M + 1))."""
    K = M + 1
    # floor(i (N+1)/K) - floor((i-1)(N+1)/K) is floor((N+1)/K) or one more
    return [((i * (N + 1)) // K) - (((i - 1) * (N + 1)) // K) for i in range(1, K + 1)]


def brute_force_optimum(p: Sequence[float], M: int, rel_tol: float = 1e-12) -> Tuple[float, List[Tuple[int, ...]]]:
    """Minimum of R over every placement of M positions in 1..N, and every
    placement that reaches it (within rel_tol).  Exponential: tiny N only."""
    N = len(p) - 1
    vals = {}
    for pos in itertools.combinations(range(1, N + 1), M):
        vals[pos] = expected_recompute(p, pos)
    best = min(vals.values())
    tol = rel_tol * max(1.0, abs(best))
    return best, [pos for pos, v in vals.items() if v <= best + tol]


def _interval_cost(p: Sequence[float], N: int) -> np.ndarray:
    """C[a][b] = sum_{d=a}^{b-1} p(d) (d - a): the recomputation of the depths
    a..b-1 served by a checkpoint (or the zero state) at a, for 0 <= a < b <= N + 1."""
    C = np.full((N + 2, N + 2), np.inf)
    for a in range(N + 1):
        acc = 0.0
        C[a][a] = 0.0
        for b in range(a + 1, N + 2):
            acc += float(p[b - 1]) * (b - 1 - a)
            C[a][b] = acc
    return C


def dp_optimum(p: Sequence[float], M: int) -> Tuple[float, List[int]]:
    """The page's recurrence (Theorem 2) in gap form, O(M N^2) with the
    interval costs tabulated term by term.  G[k][t] is the least cost of the
    depths 0..t-1 split into k gaps, the first starting at c_0 = 0 and the
    last ending at boundary t:
        G[1][t] = C(0, t),  G[k][t] = min_{s < t} G[k-1][s] + C(s, t),
    and the answer is G[M+1][N+1] (the last gap ends at the sentinel N + 1).
    Returns (cost, positions)."""
    N = len(p) - 1
    K = M + 1
    C = _interval_cost(p, N)
    G = np.full((K + 1, N + 2), np.inf)
    arg = np.zeros((K + 1, N + 2), dtype=np.int64)
    for t in range(1, N + 2):
        G[1][t] = C[0][t]
    for k in range(2, K + 1):
        for t in range(k, N + 2):
            best, bs = np.inf, -1
            for s in range(k - 1, t):
                v = G[k - 1][s] + C[s][t]
                if v < best:
                    best, bs = v, s
            G[k][t] = best
            arg[k][t] = bs
    pos = []
    t = N + 1
    for k in range(K, 1, -1):
        t = int(arg[k][t])
        pos.append(t)
    return float(G[K][N + 1]), sorted(pos)
