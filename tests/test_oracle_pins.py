"""Pins for the fp64 oracle: facts fixed by the pages or by the mathematics,
not by the oracle's own code.  CPU only.

[TR]  "Tail-Replay: Escaping the Curse of Linear Attention in Prefix Caching for Hybrid LLMs"
[SPC] "Sparse prefix caching for hybrid and recurrent LLM serving"
"""
import itertools
import json
import os

import numpy as np
import pytest

import oracle
import workloads

HERE = os.path.dirname(os.path.abspath(__file__))
FORMS = ["literal", "rank1", "c"]


def _scan(form):
    return {"literal": oracle.scan_literal, "rank1": oracle.scan_rank1,
            "c": oracle.scan_rank1_c}[form]


def _rand(rng, T, dk, dv, alpha=(0.8, 1.0), beta=(0.0, 1.0)):
    q = rng.standard_normal((T, dk))
    k = rng.standard_normal((T, dk))
    v = rng.standard_normal((T, dv))
    a = rng.uniform(*alpha, T)
    b = rng.uniform(*beta, T)
    return q, k, v, a, b


@pytest.fixture(scope="module", autouse=True)
def _c_oracle():
    from oracle.build import build_c_oracle
    if not oracle.c_oracle_available():
        build_c_oracle()


# --- single-step closed forms ------------------------------------------------

@pytest.mark.parametrize("form", FORMS)
def test_first_token_from_zero_state(form):
    """From S = 0 one step gives S_1 = beta v khat^T and o_1 = beta v (khat . qhat):
    the write term of [TR] §2.3 eq. (1) with a d_v x d_k state (d_v != d_k here
    so a transposed state cannot pass), and the output read after the update."""
    rng = np.random.default_rng(1)
    dk, dv = 5, 3
    q, k, v, a, b = _rand(rng, 1, dk, dv)
    S, O, _ = _scan(form)(np.zeros((dv, dk)), q, k, v, a, b, normalize_k=True, normalize_q=True)
    kh = k[0] / np.linalg.norm(k[0])
    qh = q[0] / np.linalg.norm(q[0])
    assert S.shape == (dv, dk)
    np.testing.assert_allclose(S, b[0] * v[0][:, None] * kh[None, :], rtol=0, atol=1e-14)
    np.testing.assert_allclose(O[0], b[0] * v[0] * float(kh @ qh), rtol=0, atol=1e-14)


@pytest.mark.parametrize("form", FORMS)
def test_delta_rule_stores_value(form):
    """alpha = 1, beta = 1, unit key: the updated state maps the key to the value,
    S_new k = v, whatever S held before (delta-rule algebra on eq. (1)).  The key
    is passed unnormalised (norm 3) to pin the fused normalisation."""
    rng = np.random.default_rng(2)
    dk, dv = 6, 4
    S0 = rng.standard_normal((dv, dk))
    k = rng.standard_normal((1, dk))
    k = 3.0 * k / np.linalg.norm(k)
    v = rng.standard_normal((1, dv))
    S, _, _ = _scan(form)(S0, None, k, v, np.ones(1), np.ones(1), normalize_k=True)
    np.testing.assert_allclose(S @ (k[0] / 3.0), v[0], rtol=0, atol=1e-13)


@pytest.mark.parametrize("form", FORMS)
def test_directions_orthogonal_to_key_untouched(form):
    """alpha = 1: the key operator acts on the d_k side only, so S x is unchanged
    for every x orthogonal to the key ([TR] §2.3: the operator right-multiplies)."""
    rng = np.random.default_rng(3)
    d = 6
    S0 = rng.standard_normal((d, d))
    k = rng.standard_normal((1, d))
    kh = k[0] / np.linalg.norm(k[0])
    x = rng.standard_normal(d)
    x -= (x @ kh) * kh
    v = rng.standard_normal((1, d))
    S, _, _ = _scan(form)(S0, None, k, v, np.ones(1), np.array([0.7]), normalize_k=True)
    np.testing.assert_allclose(S @ x, S0 @ x, rtol=0, atol=1e-13)


@pytest.mark.parametrize("form", FORMS)
def test_beta_zero(form):
    """beta = 0: alpha = 1 leaves the state bit-for-bit unchanged; otherwise the
    state is only decayed, S_T = (prod alpha) S_0."""
    rng = np.random.default_rng(4)
    d = 5
    S0 = rng.standard_normal((d, d))
    q, k, v, a, _ = _rand(rng, 7, d, d)
    S, _, _ = _scan(form)(S0, q, k, v, np.ones(7), np.zeros(7))
    if form != "literal":
        assert np.array_equal(S, S0)
    else:
        np.testing.assert_allclose(S, S0, rtol=0, atol=1e-15)
    S, _, _ = _scan(form)(S0, q, k, v, a, np.zeros(7))
    np.testing.assert_allclose(S, np.prod(a) * S0, rtol=1e-14, atol=0)


@pytest.mark.parametrize("form", FORMS)
def test_householder_reflection(form):
    """beta = 2, alpha = 1, v = 0, unit key: I - 2 k k^T is a Householder
    reflector (Golub & Van Loan, Matrix Computations, §5.1): ||S||_F is kept and
    applying the same key twice returns S."""
    rng = np.random.default_rng(5)
    d = 7
    S0 = rng.standard_normal((4, d))
    k1 = rng.standard_normal((1, d))
    k = np.concatenate([k1, k1])
    S1, _, _ = _scan(form)(S0, None, k[:1], np.zeros((1, 4)), np.ones(1), np.array([2.0]))
    assert abs(np.linalg.norm(S1) - np.linalg.norm(S0)) < 1e-13
    assert np.abs(S1 - S0).max() > 1e-3
    S2, _, _ = _scan(form)(S0, None, k, np.zeros((2, 4)), np.ones(2), np.array([2.0, 2.0]))
    np.testing.assert_allclose(S2, S0, rtol=0, atol=1e-13)


# --- multi-step closed forms -------------------------------------------------

@pytest.mark.parametrize("form", FORMS)
def test_orthonormal_keys_closed_form(form):
    """Distinct basis vectors as keys never interact, so from S_0 = 0
    S_T = sum_t (prod_{s>t} alpha_s) beta_t v_t e_t^T  (gated linear attention),
    which pins which alpha multiplies which write."""
    rng = np.random.default_rng(6)
    dk, dv, T = 8, 3, 6
    perm = rng.permutation(dk)[:T]
    k = np.eye(dk)[perm] * rng.uniform(0.5, 2.0, (T, 1))
    q = rng.standard_normal((T, dk))
    v = rng.standard_normal((T, dv))
    a = rng.uniform(0.5, 1.0, T)
    b = rng.uniform(0.1, 1.5, T)
    S, O, _ = _scan(form)(np.zeros((dv, dk)), q, k, v, a, b)
    ref = np.zeros((dv, dk))
    for t in range(T):
        ref[:, perm[t]] = np.prod(a[t + 1:]) * b[t] * v[t]
    np.testing.assert_allclose(S, ref, rtol=1e-13, atol=1e-15)
    # output after token t: the same sum truncated at t, applied to q_t
    for t in range(T):
        St = np.zeros((dv, dk))
        for s in range(t + 1):
            St[:, perm[s]] = np.prod(a[s + 1:t + 1]) * b[s] * v[s]
        np.testing.assert_allclose(O[t], St @ q[t], rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("form", FORMS)
def test_repeated_key_geometric_closed_form(form):
    """The same unit key, value, alpha and beta n times.  Along the key,
    x_t = S_t k obeys x_t = alpha (1 - beta) x_{t-1} + beta v, so
    x_n = c^n x_0 + beta v (1 - c^n)/(1 - c) with c = alpha (1 - beta);
    orthogonal to the key the state only decays, S_n y = alpha^n S_0 y."""
    rng = np.random.default_rng(7)
    d, n = 6, 9
    alpha, beta = 0.93, 0.35
    S0 = rng.standard_normal((d, d))
    k1 = rng.standard_normal(d)
    kh = k1 / np.linalg.norm(k1)
    v1 = rng.standard_normal(d)
    y = rng.standard_normal(d)
    y -= (y @ kh) * kh
    S, _, _ = _scan(form)(S0, None, np.tile(k1, (n, 1)), np.tile(v1, (n, 1)),
                          np.full(n, alpha), np.full(n, beta))
    c = alpha * (1 - beta)
    x_ref = c ** n * (S0 @ kh) + beta * v1 * (1 - c ** n) / (1 - c)
    np.testing.assert_allclose(S @ kh, x_ref, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(S @ y, alpha ** n * (S0 @ y), rtol=1e-13, atol=1e-13)


@pytest.mark.parametrize("form", FORMS)
def test_exact_split_brute_force(form):
    """[TR] §2.3 split, written with explicit products of the transitions
    P_i = alpha_i (I - beta_i k_i k_i^T) acting from the right:
      S_m = S_a P_{a+1}...P_m + sum_j b_j P_{j+1}...P_m,
    the zero-start replay equals the sum term, and the error is
    E_m = S_a P_{a+1}...P_m (empty products are the identity)."""
    rng = np.random.default_rng(8)
    dk, dv, L = 5, 4, 11
    q, k, v, a, b = _rand(rng, L, dk, dv, alpha=(0.6, 1.0), beta=(0.0, 2.0))
    kh = k / np.linalg.norm(k, axis=1, keepdims=True)
    Sa = rng.standard_normal((dv, dk))
    P = [a[i] * (np.eye(dk) - b[i] * np.outer(kh[i], kh[i])) for i in range(L)]
    prod_from = lambda i: (np.linalg.multi_dot([np.eye(dk)] + P[i:] + [np.eye(dk)]))
    E = Sa @ prod_from(0)
    Shat = sum(b[j] * np.outer(v[j], kh[j]) @ prod_from(j + 1) for j in range(L))
    S_full, _, _ = _scan(form)(Sa, q, k, v, a, b)
    S_zero, _, _ = _scan(form)(np.zeros((dv, dk)), q, k, v, a, b)
    np.testing.assert_allclose(S_zero, Shat, rtol=0, atol=1e-13)
    np.testing.assert_allclose(S_full, E + Shat, rtol=0, atol=1e-13)
    np.testing.assert_allclose(S_full - S_zero, E, rtol=0, atol=1e-13)


@pytest.mark.parametrize("form", ["rank1", "c"])
def test_contraction_bound(form):
    """[TR] §2.3: with unit keys, beta in [0, 2] and alpha_i <= rho < 1,
    ||S_m - Shat_m||_F <= rho^k ||S_a||_F over a k-token zero-start replay."""
    rng = np.random.default_rng(9)
    for trial in range(40):
        d = int(rng.integers(2, 9))
        kk = int(rng.integers(1, 65))
        rho = float(rng.uniform(0.5, 0.999))
        q, k, v, _, _ = _rand(rng, kk, d, d)
        a = rng.uniform(0.3, rho, kk)
        b = rng.uniform(0.0, 2.0, kk)
        Sa = rng.standard_normal((d, d)) * rng.uniform(0.1, 10)
        S_full, _, _ = _scan(form)(Sa, q, k, v, a, b)
        S_hat, _, _ = _scan(form)(np.zeros((d, d)), q, k, v, a, b)
        err = np.linalg.norm(S_full - S_hat)
        assert err <= rho ** kk * np.linalg.norm(Sa) * (1 + 1e-12) + 1e-300, trial
    # equality case: beta = 0 and alpha = rho everywhere gives E = rho^k S_a
    d, kk, rho = 4, 13, 0.9
    Sa = rng.standard_normal((d, d))
    q, k, v, _, _ = _rand(rng, kk, d, d)
    S_full, _, _ = _scan(form)(Sa, q, k, v, np.full(kk, rho), np.zeros(kk))
    S_hat, _, _ = _scan(form)(np.zeros((d, d)), q, k, v, np.full(kk, rho), np.zeros(kk))
    assert abs(np.linalg.norm(S_full - S_hat) - rho ** kk * np.linalg.norm(Sa)) < 1e-12


@pytest.mark.parametrize("form", FORMS)
def test_superposition(form):
    """The map (S_0, V) -> (S_T, O) is linear: scan(S_0, V) = scan(S_0, 0) + scan(0, V)
    (the affine structure behind the split of [TR] §2.3)."""
    rng = np.random.default_rng(10)
    dk, dv, T = 6, 5, 9
    q, k, v, a, b = _rand(rng, T, dk, dv)
    S0 = rng.standard_normal((dv, dk))
    f = _scan(form)
    S1, O1, _ = f(S0, q, k, v, a, b)
    S2, O2, _ = f(S0, q, k, np.zeros_like(v), a, b)
    S3, O3, _ = f(np.zeros_like(S0), q, k, v, a, b)
    np.testing.assert_allclose(S1, S2 + S3, rtol=0, atol=1e-13)
    np.testing.assert_allclose(O1, O2 + O3, rtol=0, atol=1e-13)


@pytest.mark.parametrize("form", FORMS)
def test_rows_independent(form):
    """Rows of the d_v x d_k state evolve independently ([TR] §2.3, right action):
    scanning a subset R of value channels gives rows R of S and of o."""
    rng = np.random.default_rng(11)
    dk, dv, T = 6, 7, 10
    q, k, v, a, b = _rand(rng, T, dk, dv)
    S0 = rng.standard_normal((dv, dk))
    R = [1, 4, 5]
    f = _scan(form)
    S, O, _ = f(S0, q, k, v, a, b)
    Sr, Or, _ = f(S0[R], q, k, v[:, R], a, b)
    np.testing.assert_allclose(Sr, S[R], rtol=0, atol=1e-14)
    np.testing.assert_allclose(Or, O[:, R], rtol=0, atol=1e-14)


@pytest.mark.parametrize("form", FORMS)
def test_emitted_state_is_the_state_after_that_many_tokens(form):
    """A checkpoint c holds the state after the c-th token ([SPC] §3): the state
    emitted after t tokens is the end state of the same scan over the first t
    tokens only, and the one emitted after the last token is the final state."""
    rng = np.random.default_rng(13)
    dk, dv, T = 8, 12, 20
    q, k, v, a, b = _rand(rng, T, dk, dv)
    S0 = rng.standard_normal((dv, dk))
    emit = [1, 2, 7, 20]
    S, _, st = _scan(form)(S0, q, k, v, a, b, emit_after=emit)
    assert sorted(st) == emit
    for t in emit:
        St, _, _ = _scan(form)(S0, q[:t], k[:t], v[:t], a[:t], b[:t])
        np.testing.assert_allclose(st[t], St, rtol=0, atol=1e-12)
    np.testing.assert_array_equal(st[T], S)


def test_forms_agree_and_emit_prefix_states():
    """literal, rank-1 (numpy) and rank-1 (C) agree; a state emitted after t
    tokens equals the end state of a scan over the first t tokens only."""
    rng = np.random.default_rng(12)
    dk, dv, T = 16, 16, 64
    q, k, v, a, b = _rand(rng, T, dk, dv, alpha=(0.9, 1.0), beta=(0.0, 2.0))
    S0 = rng.standard_normal((dv, dk))
    emit = [1, 16, 33, 64]
    res = [_scan(f)(S0, q, k, v, a, b, normalize_q=True, emit_after=emit) for f in FORMS]
    for r in res[1:]:
        np.testing.assert_allclose(r[0], res[0][0], rtol=0, atol=1e-12)
        np.testing.assert_allclose(r[1], res[0][1], rtol=0, atol=1e-12)
        for t in emit:
            np.testing.assert_allclose(r[2][t], res[0][2][t], rtol=0, atol=1e-12)
    for t in emit:
        St, _, _ = oracle.scan_rank1(S0, q[:t], k[:t], v[:t], a[:t], b[:t])
        assert np.array_equal(St, res[1][2][t])


# --- span selection ------------------------------------------------------------

def test_tail_worked_example_golden():
    g = json.load(open(os.path.join(HERE, "golden", "tail_worked_example.json")))
    k = oracle.tail_length(g["m"], g["r_num"], g["r_den"])
    assert k == g["k"]
    p0, n = oracle.tail_span(g["m"], g["r_num"], g["r_den"])
    assert (p0, p0 + n - 1) == (g["first_position"], g["last_position"])
    j, r0, n2 = oracle.resume_span([g["checkpoint_position"]], g["m"])
    assert (j, n2) == (1, g["exact_resume_positions"])
    assert r0 == g["checkpoint_position"] + 1


def test_tail_length_exact_rational():
    """ceil(r m) in exact integers: 5% and 10% of 32768 are 1638.4 and 3276.8."""
    assert oracle.tail_length(32768, 5, 100) == 1639
    assert oracle.tail_length(32768, 10, 100) == 3277
    assert oracle.tail_length(32768, 1, 20) == 1639
    assert oracle.tail_length(100, 5, 100) == 5       # exact: no rounding up
    assert oracle.tail_length(101, 5, 100) == 6
    assert oracle.tail_length(1, 5, 100) == 1
    assert oracle.tail_length(7, 0, 1) == 0
    assert oracle.tail_length(7, 3, 2) == 7             # r > 1 is capped at m
    for m in range(1, 400):
        for num, den in [(5, 100), (10, 100), (1, 3), (2, 7)]:
            k = oracle.tail_length(m, num, den)
            # k is the least integer with k * den >= m * num
            assert k * den >= m * num and (k - 1) * den < m * num


def test_resume_selection_gap_accounting():
    """[SPC] §3-§4: with gaps g (sum g = N + 1, checkpoints at the partial sums)
    the recompute f(d) = d - c_j summed over d = 0..N equals sum_i g_i (g_i - 1)/2
    (the phi of Theorem 1).  This fixes c_j <= d (not <), the implicit c_0 = 0,
    and zero recompute when d is itself a checkpoint."""
    rng = np.random.default_rng(13)
    for _ in range(200):
        M = int(rng.integers(0, 6))
        g = rng.integers(1, 9, size=M + 1)
        N = int(g.sum()) - 1
        pos = list(np.cumsum(g)[:M])
        total = 0
        for d in range(0, N + 1):
            j, p0, n = oracle.resume_span(pos, d)
            c = pos[j - 1] if j else 0
            assert p0 == c + 1 and n == d - c >= 0
            if d in pos:
                assert n == 0 and pos[j - 1] == d
            total += n
        assert total == sum(int(x) * (int(x) - 1) // 2 for x in g)


def test_balanced_positions_theorem1():
    """[SPC] §4 Theorem 1: for uniform d on {1..N} the optimal gaps differ by at
    most one.  Brute force over all placements for small N, M: the balanced
    placement used by the resume workload attains the minimum expected recompute."""
    def cost(pos, N):
        return sum(oracle.resume_span(list(pos), d)[2] for d in range(1, N + 1))
    for N in range(1, 13):
        for M in range(0, min(N, 4) + 1):
            best = min(cost(c, N) for c in itertools.combinations(range(1, N + 1), M))
            bal = workloads.balanced_positions(N, M)
            gaps = np.diff([0] + bal + [N + 1])
            assert gaps.max() - gaps.min() <= 1
            assert cost(bal, N) == best, (N, M)


def test_resume_from_emitted_state_equals_prefill():
    """[SPC] §3: resuming from an exact stored state S_{c_j} and recomputing
    c_j+1..d gives exactly the state of the full run at d, and the same outputs."""
    rng = np.random.default_rng(14)
    d_, N = 8, 60
    q, k, v, a, b = _rand(rng, N, d_, d_)
    pos = [7, 20, 21, 44]
    S_N, O_full, st = oracle.scan_rank1(np.zeros((d_, d_)), q, k, v, a, b,
                                        normalize_q=True, emit_after=pos + list(range(1, N + 1)))
    for depth in range(0, N + 1):
        j, p0, n = oracle.resume_span(pos, depth)
        S0 = st[pos[j - 1]] if j else np.zeros((d_, d_))
        sl = slice(p0 - 1, p0 - 1 + n)
        S, O, _ = oracle.scan_rank1(S0, q[sl], k[sl], v[sl], a[sl], b[sl], normalize_q=True)
        ref = st[depth] if depth else np.zeros((d_, d_))
        assert np.array_equal(S, ref)
        assert np.array_equal(O, O_full[sl])


def test_tail_with_k_equal_m_is_full_run():
    """r = 1: the tail is the whole prefix, so the zero-start replay is the full run."""
    rng = np.random.default_rng(15)
    m, d_ = 37, 6
    q, k, v, a, b = _rand(rng, m, d_, d_)
    p0, n = oracle.tail_span(m, 1, 1)
    assert (p0, n) == (1, m)
    S, _, _ = oracle.scan_rank1(np.zeros((d_, d_)), q, k, v, a, b)
    S2, _, _ = oracle.scan_rank1(np.zeros((d_, d_)), q[p0 - 1:], k[p0 - 1:], v[p0 - 1:],
                                 a[p0 - 1:], b[p0 - 1:])
    assert np.array_equal(S, S2)


def test_c_oracle_rejects_bad_emission_lists():
    S = np.zeros((1, 2, 2))
    k = np.ones((3, 2))
    with pytest.raises(ValueError):
        oracle.scan_rank1_c_batch([S[0]], [k], [k], [k], [np.ones(3)], [np.ones(3)],
                                  emits=[[2, 2]])
    with pytest.raises(ValueError):
        oracle.scan_rank1_c_batch([S[0]], [k], [k], [k], [np.ones(3)], [np.ones(3)],
                                  emits=[[4]])


# --- the parity metric -------------------------------------------------------------

def _rel_fro_pins(rel_fro):
    """Known answers of ||x - ref||_F / ||ref||_F, the relative Frobenius error
    every parity verdict is stated in (per (request, head) slice)."""
    ref = np.array([[3.0, 4.0]])
    # x = ref (1 + eps): the error is |eps|, whatever the sign of eps
    for eps in (1e-3, -2.5e-6, 0.5):
        assert rel_fro(ref * (1 + eps), ref) == pytest.approx(abs(eps), rel=1e-12)
    # the denominator is the reference's norm, not the result's: x = 2 ref gives 1, ref = 2 x gives 1/2
    assert rel_fro(2 * ref, ref) == pytest.approx(1.0, rel=1e-15)
    assert rel_fro(ref, 2 * ref) == pytest.approx(0.5, rel=1e-15)
    # a sign flip is an error of 2; a zero result an error of 1
    assert rel_fro(-ref, ref) == pytest.approx(2.0, rel=1e-15)
    assert rel_fro(np.zeros_like(ref), ref) == pytest.approx(1.0, rel=1e-15)
    # Frobenius over every entry of a matrix: one entry of the 3 x 3 identity off by 1 -> 1/sqrt(3)
    x = np.eye(3)
    x[2, 0] = 1.0
    assert rel_fro(x, np.eye(3)) == pytest.approx(1 / np.sqrt(3), rel=1e-15)
    # a zero reference demands an exact zero: 0 -> 0, anything else -> inf
    assert rel_fro(np.zeros((2, 2)), np.zeros((2, 2))) == 0.0
    assert rel_fro(np.array([[0.0, 1.4e-45]]), np.zeros((1, 2))) == np.inf  # the smallest float32 denormal
    # empty slices (a zero-length span) compare as equal
    assert rel_fro(np.zeros((0, 4)), np.zeros((0, 4))) == 0.0


def test_rel_fro_known_answers():
    _rel_fro_pins(oracle.rel_fro)


def _rel_fro_mutants():
    fro = lambda a: float(np.sqrt(np.sum(np.asarray(a, np.float64) ** 2)))

    def by_result(x, ref):  # divides by ||x|| instead of ||ref||
        d = fro(x)
        return fro(np.asarray(x) - ref) / d if d else (0.0 if fro(np.asarray(x) - ref) == 0 else np.inf)

    def zero_ref_passes(x, ref):  # ||ref|| = 0 reported as 0 whatever x is
        d = fro(ref)
        return fro(np.asarray(x) - ref) / d if d else 0.0

    def max_abs(x, ref):  # largest entry instead of the Frobenius norm
        d = float(np.max(np.abs(ref))) if np.size(ref) else 0.0
        n = float(np.max(np.abs(np.asarray(x) - ref))) if np.size(ref) else 0.0
        return n / d if d else (0.0 if n == 0 else np.inf)

    def squared(x, ref):  # ratio of squared norms
        d = fro(ref) ** 2
        n = fro(np.asarray(x) - ref) ** 2
        return n / d if d else (0.0 if n == 0 else np.inf)

    return {"divides by the result's norm": by_result, "zero reference always passes": zero_ref_passes,
            "max-abs instead of Frobenius": max_abs, "squared ratio": squared}


@pytest.mark.parametrize("name", list(_rel_fro_mutants()))
def test_rel_fro_mutants_fail_the_pins(name):
    """Planted mistakes in the metric (in this test, never in the oracle) each
    fail one of the known answers above."""
    with pytest.raises(AssertionError):
        _rel_fro_pins(_rel_fro_mutants()[name])
