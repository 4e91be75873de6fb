"""Helpers shared by the GPU parity tests: run the fp64 oracle on selected
(request, head) pairs of a workload and compare the library's results with it.

Tolerances (relative Frobenius error per (request, head) slice):
  float32 inputs: 1e-5     bfloat16 inputs (float32 state): 3e-3
Integers (tail lengths, selected checkpoints) must match exactly.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle
import workloads

TOL = {"f32": 1e-5, "bf16": 3e-3}


def np64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to(torch.float64).cpu().numpy()


def spans_of(w: workloads.Workload):
    """(first position, length) per request, from the oracle's integer logic."""
    if w.op == "tail":
        return [oracle.tail_span(w.m[b], w.r_num, w.r_den) for b in range(w.B)]
    if w.op == "resume":
        out = []
        for b in range(w.B):
            j, p0, n = oracle.resume_span(w.ckpt_pos[b], w.depth[b])
            out.append((p0, n))
        return out
    return [oracle.prefill_span(w.n_tokens[b]) for b in range(w.B)]


def pair_inputs(w, b, h, span, tensors=None):
    """float64 host copies of one pair's span rows."""
    q, k, v, a, bt = tensors or (w.q, w.k, w.v, w.alpha, w.beta)
    p0, n = span
    r0 = w.tok_offset[b] + (p0 - w.first_pos[b])
    sl = slice(r0, r0 + n)
    return (np64(q[sl, h]), np64(k[sl, h]), np64(v[sl, h]), np64(a[sl, h]), np64(bt[sl, h])), sl


def oracle_pairs(w, pairs, *, tensors=None, init=None, emit=None, use_c=True):
    """Run the oracle on `pairs`; returns {(b,h): (S, O, emitted dict, row slice)}."""
    spans = spans_of(w)
    fk = bool(w.flags & workloads.NORMALIZE_K)
    fq = bool(w.flags & workloads.NORMALIZE_Q)
    S0s, qs, ks, vs, als, bts, ems, slices = [], [], [], [], [], [], [], []
    for (b, h) in pairs:
        (q, k, v, a, bt), sl = pair_inputs(w, b, h, spans[b], tensors)
        S0s.append(init(b, h) if init else np.zeros((w.dv, w.dk)))
        qs.append(q); ks.append(k); vs.append(v); als.append(a); bts.append(bt)
        ems.append(emit[b] if emit else [])
        slices.append(sl)
    if use_c and oracle.c_oracle_available():
        S, O, st = oracle.scan_rank1_c_batch(S0s, qs, ks, vs, als, bts, normalize_k=fk,
                                             normalize_q=fq, emits=ems)
        return {p: (S[i], O[i], st[i], slices[i]) for i, p in enumerate(pairs)}
    res = {}
    for i, p in enumerate(pairs):
        S, O, st = oracle.scan_rank1(S0s[i], qs[i], ks[i], vs[i], als[i], bts[i],
                                     normalize_k=fk, normalize_q=fq, emit_after=ems[i])
        res[p] = (S, O, st, slices[i])
    return res


def _host(t):
    return None if t is None else t.detach().cpu()


def check_batched(w, outs, pairs=None, *, batch=64, tensors=None, init=None, emit=None, tol=None,
                  label="", log=print):
    """Compare one or more library results with the oracle on every pair of
    ``pairs`` (default: all (request, head) pairs), running the C oracle on
    ``batch`` pairs at a time so that full-size workloads fit in host memory.

    outs: {name: (state_out, o or None, ckpt or None)} of device tensors.
    Returns {name: worst errors}."""
    pairs = [(b, h) for b in range(w.B) for h in range(w.H)] if pairs is None else list(pairs)
    q, k, v, a, bt = tensors or (w.q, w.k, w.v, w.alpha, w.beta)
    host = workloads.Workload(**{**w.__dict__, "q": _host(q), "k": _host(k), "v": _host(v),
                                 "alpha": _host(a), "beta": _host(bt)})
    h_outs = {n: tuple(_host(t) for t in ts) for n, ts in outs.items()}
    worst = {n: {"state": 0.0, "o": 0.0, "emit": 0.0} for n in outs}
    for i in range(0, len(pairs), batch):
        sel = pairs[i:i + batch]
        ref = oracle_pairs(host, sel, init=init, emit=emit)
        for n, (S, O, C) in h_outs.items():
            got = compare(host, ref, S, O, C, tol=tol, label=f"{label}[{n}]")
            for key in got:
                worst[n][key] = max(worst[n][key], got[key])
        del ref
    log(f"[{label}] {len(pairs)} pairs, worst rel err {worst}")
    return worst


def init_for(w):
    """Start state per pair for a resume workload (None: zero start)."""
    if w.op != "resume":
        return None
    ck = w.ckpt_states

    def f(b, h):
        j = oracle.select_checkpoint(w.ckpt_pos[b], w.depth[b])
        if j == 0:
            return np.zeros((w.dv, w.dk))
        return np64(ck[b, j - 1, h])
    return f


def emit_for(w):
    if w.op != "prefill":
        return None
    return [list(p) for p in w.ckpt_pos]


def compare(w, ref, state_out, o, ckpt_out=None, tol=None, label=""):
    """Assert parity on every pair in `ref`; returns the worst errors seen."""
    tol = TOL[w.dtype] if tol is None else tol
    worst = {"state": 0.0, "o": 0.0, "emit": 0.0}
    for (b, h), (S, O, st, sl) in ref.items():
        e = oracle.rel_fro(np64(state_out[b, h]), S)
        worst["state"] = max(worst["state"], e)
        assert e <= tol, f"{label} state (b={b}, h={h}): rel err {e:.3g} > {tol}"
        if o is not None and O is not None and O.shape[0] > 0:
            e = oracle.rel_fro(np64(o[sl, h]), O)
            worst["o"] = max(worst["o"], e)
            assert e <= tol, f"{label} output (b={b}, h={h}): rel err {e:.3g} > {tol}"
        if ckpt_out is not None:
            for i, c in enumerate(w.ckpt_pos[b]):
                e = oracle.rel_fro(np64(ckpt_out[b, i, h]), st[c])
                worst["emit"] = max(worst["emit"], e)
                assert e <= tol, f"{label} emitted state {i} at {c} (b={b}, h={h}): {e:.3g} > {tol}"
    return worst


def run_library(gdn, w, *, flags_extra=0, want_o=True, o=None, state_out=None):
    """Call the library entry point matching the workload."""
    flags = w.flags | flags_extra
    if w.op == "tail":
        S, O, ks = gdn.tail_replay(w.q, w.k, w.v, w.alpha, w.beta, w.tok_offset, w.m,
                                   w.r_num, w.r_den, first_pos=w.first_pos, flags=flags,
                                   want_o=want_o, o=o, state_out=state_out)
        return dict(state=S, o=O, k=ks)
    if w.op == "resume":
        S, O, js = gdn.resume(w.q, w.k, w.v, w.alpha, w.beta, w.tok_offset, w.ckpt_pos,
                              w.ckpt_states, w.depth, first_pos=w.first_pos, flags=flags,
                              want_o=want_o, o=o, state_out=state_out)
        return dict(state=S, o=O, j=js)
    C, S, O = gdn.prefill_emit_checkpoints(w.q, w.k, w.v, w.alpha, w.beta, w.tok_offset,
                                           w.ckpt_pos, flags=flags, want_o=want_o, o=o,
                                           state_out=state_out)
    return dict(state=S, o=O, ckpt=C)


def to_device(w, device="cuda"):
    for name in ("q", "k", "v", "alpha", "beta", "ckpt_states"):
        t = getattr(w, name)
        if t is not None:
            setattr(w, name, t.to(device))
    if w.layer_alpha:
        w.layer_alpha = [t.to(device) for t in w.layer_alpha]
        w.layer_beta = [t.to(device) for t in w.layer_beta]
    return w
