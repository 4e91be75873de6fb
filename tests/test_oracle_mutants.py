"""The oracle's pins catch plausible mistakes: each mutant below is the rank-1
scan with one mistake of the kind a reader of "Tail-Replay: Escaping the Curse
of Linear Attention in Prefix Caching for Hybrid LLMs" §2.3 eq. (1) could make
(a dropped or misplaced decay, a wrong sign, a dropped beta, a transposed write,
the output taken before the update, the key left unnormalised, the state
recorded before the update).  Every parametrised pin of test_oracle_pins.py is
run with the mutant in place of the scan, and at least one of them must fail.
The same holds for mistakes in the span selection ([TR] §2.1-§2.2, [SPC] §3:
the tail length, the replayed range, the checkpoint chosen for a depth).
And for the checkpoint-placement oracle ("Sparse prefix caching for hybrid and
recurrent LLM serving" §3-§4: the recompute f_g(d), the DP interval costs,
the balanced gaps), against the pins of test_planner.py.
The mistakes are planted here, in CPU test code, never in the oracle's files;
the integer ones replace an oracle function only for the duration of a test."""
import importlib.util
import os

import numpy as np
import pytest

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))


def _load_pins():
    spec = importlib.util.spec_from_file_location("_pins_for_mutants", os.path.join(HERE, "test_oracle_pins.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def _unit(x):
    x = np.asarray(x, np.float64)
    n = np.linalg.norm(x, axis=-1, keepdims=True)
    return np.where(n > 0, x / np.where(n > 0, n, 1.0), 0.0)


def _mutant(step, *, out_before=False, normalize=True, emit_before=False):
    """A rank-1 scan whose per-token update is ``step(S, a, b, k, v)``."""
    def scan(S0, q, k, v, alpha, beta, *, normalize_k=True, normalize_q=False, emit_after=()):
        S = np.array(S0, dtype=np.float64, copy=True)
        kh = _unit(k) if (normalize_k and normalize) else np.asarray(k, np.float64)
        qh = None if q is None else (_unit(q) if normalize_q else np.asarray(q, np.float64))
        v = np.asarray(v, np.float64)
        emit = set(int(t) for t in emit_after)
        out = np.zeros((kh.shape[0], S.shape[0])) if qh is not None else None
        states = {}
        for t in range(kh.shape[0]):
            prev = S
            if emit_before and (t + 1) in emit:
                states[t + 1] = S.copy()
            S = step(S, float(alpha[t]), float(beta[t]), kh[t], v[t])
            if out is not None:
                out[t] = (prev if out_before else S) @ qh[t]
            if not emit_before and (t + 1) in emit:
                states[t + 1] = S.copy()
        return S, out, states
    return scan


def _ok(S, a, b, k, v):
    return a * S + np.outer(b * (v - a * (S @ k)), k)


MUTANTS = {
    "correction without decay": _mutant(lambda S, a, b, k, v: a * S + np.outer(b * (v - S @ k), k)),
    "decay on the write too": _mutant(lambda S, a, b, k, v: a * (S + np.outer(b * (v - S @ k), k))),
    "wrong sign of the correction": _mutant(lambda S, a, b, k, v: a * S + np.outer(b * (v + a * (S @ k)), k)),
    "beta dropped from the write": _mutant(lambda S, a, b, k, v: a * S + np.outer(v - a * b * (S @ k), k)),
    "beta squared": _mutant(lambda S, a, b, k, v: a * S + np.outer(b * b * (v - a * (S @ k)), k)),
    "transposed write": _mutant(lambda S, a, b, k, v: a * S + np.outer(b * (v - a * (S @ k)), k).T.reshape(S.shape)),
    # left multiplication only type-checks for a square state
    "key operator from the left": _mutant(
        lambda S, a, b, k, v: (a * (np.eye(len(k)) - b * np.outer(k, k)) @ S + b * np.outer(v, k))
        if S.shape[0] == S.shape[1] else np.full_like(S, np.nan)),
    "output before the update": _mutant(_ok, out_before=True),
    "key left unnormalised": _mutant(_ok, normalize=False),
    "state recorded before the update": _mutant(_ok, emit_before=True),
}


def _form_pins(P):
    """The pins parametrised by the scan form (the ones a mutant scan can replace)."""
    names = [n for n in dir(P) if n.startswith("test_")]
    out = []
    for n in names:
        fn = getattr(P, n)
        marks = getattr(fn, "pytestmark", [])
        if any(m.name == "parametrize" and m.args and m.args[0] == "form" for m in marks):
            out.append(fn)
    return out


@pytest.fixture(scope="module", autouse=True)
def _c_oracle():
    from oracle.build import build_c_oracle
    if not oracle.c_oracle_available():
        build_c_oracle()


def test_the_correct_scan_passes_every_pin(monkeypatch):
    """Control: the same harness with the correct step fails no pin."""
    P = _load_pins()
    good = _mutant(_ok)
    monkeypatch.setattr(P, "_scan", lambda form: good)
    pins = _form_pins(P)
    assert len(pins) >= 8
    for fn in pins:
        fn("rank1")


@pytest.mark.parametrize("name", list(MUTANTS))
def test_every_mutant_fails_a_pin(name, monkeypatch):
    P = _load_pins()
    monkeypatch.setattr(P, "_scan", lambda form: MUTANTS[name])
    caught = []
    for fn in _form_pins(P):
        try:
            with np.errstate(all="ignore"):
                fn("rank1")
        except (AssertionError, ValueError, IndexError):
            caught.append(fn.__name__)
    assert caught, f"mutant '{name}' passes every pin"


# ---- span selection: integer mistakes -----------------------------------------

def _first_at_or_after(positions, depth):
    for i, c in enumerate(positions, start=1):
        if int(c) >= int(depth):
            return i
    return 0


def _strictly_before(positions, depth):
    j = 0
    for i, c in enumerate(positions, start=1):
        if int(c) < int(depth):
            j = i
    return j


INT_MUTANTS = {
    "tail length by floor": {"tail_length": lambda m, rn, rd: max(0, min((int(m) * int(rn)) // int(rd), int(m)))},
    "tail length by float rounding": {"tail_length": lambda m, rn, rd: max(0, min(int(round(m * rn / rd)), int(m)))},
    "tail span starts one early": {"tail_span": lambda m, rn, rd: (m - oracle.tail_length(m, rn, rd), oracle.tail_length(m, rn, rd))},
    "tail span one token short": {"tail_span": lambda m, rn, rd: (m - oracle.tail_length(m, rn, rd) + 1, max(0, oracle.tail_length(m, rn, rd) - 1))},
    "checkpoint strictly before the depth": {"select_checkpoint": _strictly_before},
    "first checkpoint at or after the depth": {"select_checkpoint": _first_at_or_after},
    "resume span includes the checkpoint token": {"resume_span": lambda pos, d: (
        oracle.select_checkpoint(pos, d),
        (int(pos[oracle.select_checkpoint(pos, d) - 1]) if oracle.select_checkpoint(pos, d) else 0),
        int(d) - (int(pos[oracle.select_checkpoint(pos, d) - 1]) if oracle.select_checkpoint(pos, d) else 0) + 1)},
}


def _all_pins(P):
    """Every pin callable here: no arguments, or only the scan form."""
    import inspect
    out = []
    for n in dir(P):
        if not n.startswith("test_"):
            continue
        fn = getattr(P, n)
        params = list(inspect.signature(fn).parameters)
        if params == []:
            out.append((fn, ()))
        elif params == ["form"]:
            out.append((fn, ("rank1",)))
    return out


def test_the_correct_span_logic_passes_every_pin():
    P = _load_pins()
    pins = _all_pins(P)
    assert len(pins) >= 15
    for fn, args in pins:
        fn(*args)


@pytest.mark.parametrize("name", list(INT_MUTANTS))
def test_every_span_mutant_fails_a_pin(name, monkeypatch):
    for attr, fn in INT_MUTANTS[name].items():
        monkeypatch.setattr(oracle, attr, fn)
    P = _load_pins()
    caught = []
    for fn, args in _all_pins(P):
        try:
            fn(*args)
        except (AssertionError, ValueError, IndexError):
            caught.append(fn.__name__)
    assert caught, f"mutant '{name}' passes every pin"


# ---- checkpoint placement: mistakes in the planner oracle ---------------------

def _load_planner_pins():
    spec = importlib.util.spec_from_file_location("_planner_pins_for_mutants", os.path.join(HERE, "test_planner.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def _recompute_counting_the_checkpoint(positions, d):
    if d == 0:
        return 0
    best = max([0] + [int(c) for c in positions if int(c) <= d])
    return d - best + 1


def _recompute_strictly_before(positions, d):
    if d == 0:
        return 0
    return d - max([0] + [int(c) for c in positions if int(c) < d])


def _interval_cost_off_by_one(p, N):
    C = np.full((N + 2, N + 2), np.inf)
    for a in range(N + 1):
        acc = 0.0
        C[a][a] = 0.0
        for b in range(a + 1, N + 2):
            acc += float(p[b - 1]) * (b - a)
            C[a][b] = acc
    return C


def _balanced_without_sentinel(N, M):
    K = M + 1
    return [((i * N) // K) - (((i - 1) * N) // K) for i in range(1, K + 1)]


PLANNER_MUTANTS = {
    "the checkpoint token is recomputed": {"recompute_len": _recompute_counting_the_checkpoint},
    "resume only from checkpoints strictly before the depth": {"recompute_len": _recompute_strictly_before},
    "interval cost counts one token too many": {"_interval_cost": _interval_cost_off_by_one},
    "balanced gaps sum to N instead of N + 1": {"balanced_gaps": _balanced_without_sentinel},
}


def _argless_pins(P):
    import inspect
    return [getattr(P, n) for n in dir(P)
            if n.startswith("test_") and not inspect.signature(getattr(P, n)).parameters]


def test_the_correct_planner_oracle_passes_every_pin():
    pins = _argless_pins(_load_planner_pins())
    assert len(pins) >= 8
    for fn in pins:
        fn()


@pytest.mark.parametrize("name", list(PLANNER_MUTANTS))
def test_every_planner_mutant_fails_a_pin(name, monkeypatch):
    from oracle import planner as OPM
    for attr, fn in PLANNER_MUTANTS[name].items():
        monkeypatch.setattr(OPM, attr, fn)
    caught = []
    for fn in _argless_pins(_load_planner_pins()):
        try:
            fn()
        except (AssertionError, ValueError, IndexError):
            caught.append(fn.__name__)
    assert caught, f"mutant '{name}' passes every pin"
