"""fp64 CPU oracle for Gated DeltaNet span replay.

TEST INFRASTRUCTURE ONLY.  This package is the slow, plain definition that the
GPU library is checked against.  Only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` may import it.  The product path
(``gated_delta_rule_scan_amd``) never imports, links or calls anything here,
and nothing here imports the product path.

Sources (cited by title and section):
  [TR]  "Tail-Replay: Escaping the Curse of Linear Attention in Prefix Caching
        for Hybrid LLMs" (notes page on arXiv 2608.30310v2).
  [SPC] "Sparse prefix caching for hybrid and recurrent LLM serving"
        (arXiv 2605.05219, translated page).

What is computed (all arithmetic in float64):
  * the state recurrence of [TR] §2.3 eq. (1), with the state S stored as a
    d_v x d_k matrix and the key operator acting from the right, as [TR] §2.3
    requires for a rectangular state:
        S_i = alpha_i * S_{i-1} (I - beta_i k_i k_i^T) + beta_i v_i k_i^T
  * the per-token output o_i = S_i q_i, read from the post-update state (the
    pages never define an output; this is the plainest reading);
  * optional exact L2 normalisation of k (and q) before use, k/||k||, with a
    zero row kept at zero (no epsilon);
  * span selection: resume from the deepest checkpoint c_j <= d ([SPC] §3),
    zero-start tail replay of the last k = ceil(r*m) positions ([TR] §2.1
    symbol table and §2.2), full prefill 1..N with states emitted at the
    checkpoint positions ([SPC] §3: a state is kept at every checkpoint).

Two forms of the scan are provided:
  ``scan_literal``  builds the d_k x d_k transition T_i = alpha_i (I - beta_i k k^T)
                    explicitly and applies S <- S T_i + beta_i v k^T;
  ``scan_rank1``    the same step written as S <- alpha S + beta (v - alpha S k) k^T.
Both are pinned by the tests in ``tests/test_oracle_pins.py`` against facts
the pages and the mathematics fix (closed forms, the exact split of [TR] §2.3,
the contraction bound of [TR] §2.3, Householder special cases, brute force).

The C form in ``gdn_oracle.c`` (``scan_rank1_c``) is the rank-1 form compiled
with OpenMP over (request, head) pairs, for large sampled checks and for the
CPU baseline timing; it is pinned against ``scan_rank1``.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Iterable, Sequence

import numpy as np

__all__ = [
    "normalize_rows",
    "transition_matrix",
    "write_term",
    "scan_literal",
    "scan_rank1",
    "tail_length",
    "select_checkpoint",
    "tail_span",
    "resume_span",
    "prefill_span",
    "scan_rank1_c",
    "c_oracle_available",
    "rel_fro",
]

# ---------------------------------------------------------------------------
# elementary pieces of [TR] §2.3 eq. (1)
# ---------------------------------------------------------------------------


def normalize_rows(x: np.ndarray) -> np.ndarray:
    """Exact L2 normalisation x/||x||_2 of each row in float64; zero rows stay 0."""
    x = np.asarray(x, dtype=np.float64)
    n = np.sqrt(np.sum(x * x, axis=-1, keepdims=True))
    out = np.zeros_like(x)
    np.divide(x, n, out=out, where=n > 0)
    return out


def transition_matrix(alpha: float, beta: float, khat: np.ndarray) -> np.ndarray:
    """T = alpha (I - beta k k^T), the key-space operator of [TR] §2.3 eq. (1)."""
    khat = np.asarray(khat, dtype=np.float64)
    dk = khat.shape[0]
    return alpha * (np.eye(dk) - beta * np.outer(khat, khat))


def write_term(beta: float, v: np.ndarray, khat: np.ndarray) -> np.ndarray:
    """b = beta v k^T, the write of [TR] §2.3 eq. (1), shape d_v x d_k."""
    return beta * np.outer(np.asarray(v, np.float64), np.asarray(khat, np.float64))


def _prep(q, k, normalize_k: bool, normalize_q: bool):
    k = np.asarray(k, dtype=np.float64)
    q = None if q is None else np.asarray(q, dtype=np.float64)
    kh = normalize_rows(k) if normalize_k else k
    qh = None if q is None else (normalize_rows(q) if normalize_q else q)
    return qh, kh


def scan_literal(S0, q, k, v, alpha, beta, *, normalize_k=True, normalize_q=False,
                 emit_after: Iterable[int] = ()):
    """Scan a span with explicit transition matrices.

    S0: (d_v, d_k) initial state.  q, k: (T, d_k); v: (T, d_v); alpha, beta: (T,).
    emit_after: token counts t in 1..T after which the state is recorded.
    Returns (S_T, O with O[t] = S_{t+1} q_{t+1}, {t: S_t}).
    """
    S = np.array(S0, dtype=np.float64, copy=True)
    qh, kh = _prep(q, k, normalize_k, normalize_q)
    v = np.asarray(v, np.float64)
    T = kh.shape[0]
    emit = set(int(t) for t in emit_after)
    out = np.zeros((T, S.shape[0])) if qh is not None else None
    states = {}
    for t in range(T):
        S = S @ transition_matrix(float(alpha[t]), float(beta[t]), kh[t]) \
            + write_term(float(beta[t]), v[t], kh[t])
        if out is not None:
            out[t] = S @ qh[t]
        if (t + 1) in emit:
            states[t + 1] = S.copy()
    return S, out, states


def scan_rank1(S0, q, k, v, alpha, beta, *, normalize_k=True, normalize_q=False,
               emit_after: Iterable[int] = ()):
    """Same scan as ``scan_literal`` in rank-1 form:
    S <- alpha S + beta (v - alpha S k) k^T  (expands [TR] §2.3 eq. (1))."""
    S = np.array(S0, dtype=np.float64, copy=True)
    qh, kh = _prep(q, k, normalize_k, normalize_q)
    v = np.asarray(v, np.float64)
    T = kh.shape[0]
    emit = set(int(t) for t in emit_after)
    out = np.zeros((T, S.shape[0])) if qh is not None else None
    states = {}
    for t in range(T):
        a = float(alpha[t])
        w = float(beta[t]) * (v[t] - a * (S @ kh[t]))
        S = a * S + np.outer(w, kh[t])
        if out is not None:
            out[t] = S @ qh[t]
        if (t + 1) in emit:
            states[t + 1] = S.copy()
    return S, out, states


# ---------------------------------------------------------------------------
# span selection: integer logic, exact
# ---------------------------------------------------------------------------


def tail_length(m: int, r_num: int, r_den: int) -> int:
    """k = ceil(r*m) with r = r_num/r_den, in exact integers, kept within [0, m].

    [TR] §2.1 symbol table defines k = ceil(r m) as the number of replayed
    tokens; §2.2 works the example m = 10000, r = 5% -> positions 9501..10000.
    """
    m, r_num, r_den = int(m), int(r_num), int(r_den)
    if r_den <= 0 or r_num < 0 or m < 0:
        raise ValueError("tail_length: need m >= 0, r_num >= 0, r_den > 0")
    k = -((-m * r_num) // r_den)  # ceiling division of non-negative integers
    return max(0, min(k, m))


def select_checkpoint(positions: Sequence[int], depth: int) -> int:
    """j = the 1-based index of the deepest checkpoint c_j <= depth, 0 if none.

    [SPC] §3: resume from argmax{c_i : c_i <= d}; when no checkpoint lies at or
    before d the recomputation starts from the zero state (implicit c_0 = 0),
    which is what the gap accounting sum(g) = N+1 of [SPC] §3 implies.
    """
    j = 0
    for i, c in enumerate(positions, start=1):
        if int(c) <= int(depth):
            j = i
    return j


def tail_span(m: int, r_num: int, r_den: int):
    """(first position, length) of the zero-start replay: m-k+1 .. m ([TR] §2.2)."""
    k = tail_length(m, r_num, r_den)
    return m - k + 1, k


def resume_span(positions: Sequence[int], depth: int):
    """(j, first position, length): recompute c_j+1 .. d from S_{c_j} ([SPC] §3)."""
    j = select_checkpoint(positions, depth)
    c = int(positions[j - 1]) if j > 0 else 0
    return j, c + 1, int(depth) - c


def prefill_span(n_tokens: int):
    """(first position, length) of the full prefill 1..N."""
    return 1, int(n_tokens)


def rel_fro(x, ref) -> float:
    """Relative Frobenius error ||x - ref||_F / ||ref||_F (exact 0 required if ref == 0)."""
    x = np.asarray(x, np.float64)
    ref = np.asarray(ref, np.float64)
    den = float(np.sqrt(np.sum(ref * ref)))
    num = float(np.sqrt(np.sum((x - ref) ** 2)))
    if den == 0.0:
        return 0.0 if num == 0.0 else math.inf
    return num / den


# ---------------------------------------------------------------------------
# the C rank-1 form (gdn_oracle.c), loaded with ctypes
# ---------------------------------------------------------------------------

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libgdn_oracle.so")
_lib = None


def _load_c():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(
                f"C oracle not built ({_LIB_PATH}); run oracle.build.build_c_oracle()")
        lib = ctypes.CDLL(_LIB_PATH)
        P = ctypes.POINTER
        d = ctypes.c_double
        i64 = ctypes.c_int64
        lib.gdn_oracle_scan_batch.argtypes = [
            ctypes.c_int32, P(i64), ctypes.c_int32, ctypes.c_int32,
            P(d), P(d), P(d), P(d), P(d), ctypes.c_int32, ctypes.c_int32,
            P(d), P(d), P(i64), P(i64), P(d), ctypes.c_int32]
        lib.gdn_oracle_scan_batch.restype = ctypes.c_int32
        lib.gdn_oracle_threads.argtypes = []
        lib.gdn_oracle_threads.restype = ctypes.c_int32
        _lib = lib
    return _lib


def c_oracle_available() -> bool:
    return os.path.exists(_LIB_PATH)


def _dptr(a):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def _iptr(a):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_int64))


def scan_rank1_c_batch(S0s, qs, ks, vs, alphas, betas, *, normalize_k=True,
                       normalize_q=False, emits=None, want_o=True, threads=0):
    """Batch form of the C oracle.  All per-pair arguments are lists of arrays.

    Returns (final states [P,d_v,d_k], list of O arrays or None, list of dicts).
    ``threads`` = 0 uses the OpenMP default.
    """
    lib = _load_c()
    P = len(ks)
    dv, dk = np.asarray(S0s[0]).shape
    lens = np.array([np.asarray(kk).shape[0] for kk in ks], dtype=np.int64)
    off = np.zeros(P + 1, np.int64)
    off[1:] = np.cumsum(lens)
    cat = lambda xs, w: (np.ascontiguousarray(np.concatenate(
        [np.asarray(x, np.float64).reshape(-1, w) for x in xs], axis=0))
        if off[-1] > 0 else np.zeros((0, w)))
    qc = cat(qs, dk) if want_o else np.zeros((0, dk))
    kc = cat(ks, dk)
    vc = cat(vs, dv)
    ac = cat(alphas, 1).reshape(-1)
    bc = cat(betas, 1).reshape(-1)
    S = np.ascontiguousarray(np.stack([np.asarray(s, np.float64) for s in S0s]))
    O = np.zeros((int(off[-1]), dv)) if want_o else None
    emits = emits if emits is not None else [()] * P
    eoff = np.zeros(P + 1, np.int64)
    eoff[1:] = np.cumsum([len(list(e)) for e in emits])
    eafter = np.array([int(t) for e in emits for t in e], dtype=np.int64)
    if eafter.size == 0:
        eafter = np.zeros(1, np.int64)
    ES = np.zeros((max(int(eoff[-1]), 1), dv, dk))
    null_d = ctypes.POINTER(ctypes.c_double)()
    rc = lib.gdn_oracle_scan_batch(
        P, _iptr(off), dk, dv,
        _dptr(qc) if want_o else null_d, _dptr(kc), _dptr(vc), _dptr(ac), _dptr(bc),
        int(bool(normalize_k)), int(bool(normalize_q)),
        _dptr(S), _dptr(O) if want_o else null_d,
        _iptr(eoff), _iptr(eafter), _dptr(ES), int(threads))
    if rc != 0:
        raise ValueError(f"C oracle rejected its arguments (code {rc})")
    outs = [O[off[p]:off[p + 1]] for p in range(P)] if want_o else None
    st = []
    for p in range(P):
        e = list(emits[p])
        st.append({int(t): ES[eoff[p] + i].copy() for i, t in enumerate(e)})
    return S, outs, st


def scan_rank1_c(S0, q, k, v, alpha, beta, *, normalize_k=True, normalize_q=False,
                 emit_after: Iterable[int] = ()):
    """Single-pair wrapper of the C rank-1 oracle with the signature of ``scan_rank1``."""
    want_o = q is not None
    S, outs, st = scan_rank1_c_batch(
        [S0], [q if want_o else np.zeros((np.asarray(k).shape[0], np.asarray(k).shape[1]))],
        [k], [v], [alpha], [beta], normalize_k=normalize_k, normalize_q=normalize_q,
        emits=[list(emit_after)], want_o=want_o)
    return S[0], (outs[0] if want_o else None), st[0]


def c_oracle_threads() -> int:
    return int(_load_c().gdn_oracle_threads())
