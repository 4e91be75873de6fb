"""Seeded synthetic inputs for Gated DeltaNet span replay.

This module only draws and lays out inputs; it holds none of the replay
arithmetic, and it is shared by the tests, the smoke check and the benchmark
(both the GPU path and the CPU oracle read the tensors it returns).

Packed layout (shared by every operation):
  q, k   [rows][H][d_k]     v   [rows][H][d_v]     alpha, beta   [rows][H]
  request b owns rows tok_offset[b] .. tok_offset[b+1]-1, and row tok_offset[b]
  holds the token at 1-based position first_pos[b] of that request.

Value recipe (the same for every workload unless a field says otherwise):
  q, k ~ N(0, 1) per element, then each row divided by its L2 norm (unit keys
  and queries), v ~ N(0, 1), alpha ~ U[alpha_lo, alpha_hi], beta ~ U[0, beta_hi),
  all drawn in float32 from a seeded torch generator on the target device and
  cast (round to nearest even) to the workload dtype.  Checkpoint states are
  N(0, 0.05^2) float32.  Integer metadata (depths, checkpoint positions) comes
  from numpy's PCG64 with the same seed and does not depend on the device.

Rows outside every span can be filled with NaN ("poison") so that a read
outside the span shows up in the results.
"""
from __future__ import annotations

import dataclasses
from typing import List, Optional

import numpy as np
import torch

NORMALIZE_K = 1
NORMALIZE_Q = 2


@dataclasses.dataclass
class Workload:
    name: str
    op: str                      # "prefill" | "resume" | "tail"
    B: int
    H: int
    dk: int
    dv: int
    dtype: str                   # "f32" | "bf16"
    flags: int
    q: torch.Tensor
    k: torch.Tensor
    v: torch.Tensor
    alpha: torch.Tensor
    beta: torch.Tensor
    tok_offset: List[int]
    first_pos: List[int]
    n_tokens: List[int]          # N_b: the request's prefix length
    # tail replay
    m: Optional[List[int]] = None
    r_num: int = 0
    r_den: int = 1
    # resume / prefill emission
    ckpt_pos: Optional[List[List[int]]] = None
    ckpt_states: Optional[torch.Tensor] = None
    depth: Optional[List[int]] = None
    # grouped tail replay: per-layer alpha/beta for layers 2.. (layer 1 uses alpha/beta)
    layers: int = 1
    layer_alpha: Optional[List[torch.Tensor]] = None
    layer_beta: Optional[List[torch.Tensor]] = None
    seed: int = 0

    @property
    def torch_dtype(self):
        return torch.float32 if self.dtype == "f32" else torch.bfloat16

    @property
    def rows(self) -> int:
        return self.tok_offset[-1]


def _tdtype(dtype: str):
    return torch.float32 if dtype == "f32" else torch.bfloat16


def _unit_rows(x: torch.Tensor) -> torch.Tensor:
    return x / torch.linalg.vector_norm(x, dim=-1, keepdim=True)


def _draw_tokens(g, rows, H, dk, dv, dtype, device, alpha_rng, beta_hi):
    td = _tdtype(dtype)
    q = _unit_rows(torch.randn(rows, H, dk, generator=g, device=device)).to(td)
    k = _unit_rows(torch.randn(rows, H, dk, generator=g, device=device)).to(td)
    v = torch.randn(rows, H, dv, generator=g, device=device).to(td)
    lo, hi = alpha_rng
    alpha = (lo + (hi - lo) * torch.rand(rows, H, generator=g, device=device)).to(td)
    beta = (beta_hi * torch.rand(rows, H, generator=g, device=device)).to(td)
    return q, k, v, alpha, beta


def _gen(device, seed):
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def _offsets(lengths):
    off = [0]
    for n in lengths:
        off.append(off[-1] + int(n))
    return off


def tiny_prefill(device="cpu", seed=1):
    """1 request, 1 head, d_k = d_v = 16, T = 64, float32, zero start, states
    emitted after 16, 32, 48 and 64 tokens."""
    return prefill(device=device, seed=seed, B=1, H=1, d=16, N=64, M=4, dtype="f32",
                   alpha_rng=(0.9, 1.0), beta_hi=1.0, positions=[[16, 32, 48, 64]],
                   name="tiny_prefill_emit_d16_T64_f32")


def prefill(device="cpu", seed=5, B=4, H=32, d=128, N=65536, M=16, dtype="bf16",
            alpha_rng=(0.9, 1.0), beta_hi=2.0, positions=None, lengths=None, name=None):
    """Full prefill of N tokens per request from the zero state, emitting states
    at M sorted distinct positions per request drawn without replacement from
    [1, N] (independently per request)."""
    rng = np.random.default_rng(seed)
    lengths = [N] * B if lengths is None else list(lengths)
    if positions is None:
        positions = []
        for b in range(B):
            n_b = lengths[b]
            mm = min(M, n_b)
            positions.append(sorted(int(x) + 1 for x in rng.choice(n_b, size=mm, replace=False)))
    off = _offsets(lengths)
    g = _gen(device, seed)
    q, k, v, a, bt = _draw_tokens(g, off[-1], H, d, d, dtype, device, alpha_rng, beta_hi)
    return Workload(name=name or f"prefill_emit_B{B}_H{H}_N{N}_M{M}", op="prefill", B=B, H=H,
                    dk=d, dv=d, dtype=dtype, flags=NORMALIZE_K | NORMALIZE_Q,
                    q=q, k=k, v=v, alpha=a, beta=bt, tok_offset=off, first_pos=[1] * B,
                    n_tokens=lengths, ckpt_pos=positions, seed=seed)


def balanced_positions(N: int, M: int) -> List[int]:
    """M checkpoints whose M+1 gaps (with the implicit start 0 and end N+1)
    differ by at most one: c_i = floor(i (N+1) / (M+1))."""
    return [(i * (N + 1)) // (M + 1) for i in range(1, M + 1)]


def resume(device="cpu", seed=2, B=8, H=16, d=128, N=8192, M=8, dtype="bf16",
           alpha_rng=(0.9, 1.0), beta_hi=1.0, depths=None, state_std=0.05, name=None):
    """Resume from the deepest stored checkpoint at or before an overlap depth
    d ~ U{1..N}: the full N-token prefix is stored per request, M balanced
    checkpoint positions, stored states N(0, state_std^2) in float32 laid out
    [B][M][H][d_v][d_k]."""
    rng = np.random.default_rng(seed)
    pos = balanced_positions(N, M)
    if depths is None:
        depths = [int(x) for x in rng.integers(1, N + 1, size=B)]
    off = _offsets([N] * B)
    g = _gen(device, seed)
    q, k, v, a, bt = _draw_tokens(g, off[-1], H, d, d, dtype, device, alpha_rng, beta_hi)
    ck = state_std * torch.randn(B, M, H, d, d, generator=g, device=device)
    return Workload(name=name or f"resume_B{B}_H{H}_N{N}_M{M}", op="resume", B=B, H=H,
                    dk=d, dv=d, dtype=dtype, flags=NORMALIZE_K | NORMALIZE_Q,
                    q=q, k=k, v=v, alpha=a, beta=bt, tok_offset=off, first_pos=[1] * B,
                    n_tokens=[N] * B, ckpt_pos=[list(pos) for _ in range(B)],
                    ckpt_states=ck, depth=depths, seed=seed)


def _ceil_div(a, b):
    return -((-a) // b)


def tail(device="cpu", seed=3, B=16, H=32, d=128, m=32768, r_num=5, r_den=100,
         dtype="bf16", alpha_rng=(0.95, 1.0), beta_hi=1.0, layers=1, pad=0, m_list=None,
         name=None):
    """Zero-start tail replay of the last ceil(r m) of m matched tokens.  Only
    the tail rows (plus ``pad`` extra rows on each side, for poisoning) are
    stored: first_pos[b] = m - ceil(r m) + 1 - pad.  With layers > 1 fresh
    alpha/beta are drawn for each further layer (grouped replay)."""
    m_list = [m] * B if m_list is None else list(m_list)
    ks = [min(m_b, _ceil_div(m_b * r_num, r_den)) for m_b in m_list]
    first = [max(1, m_b - k_b + 1 - pad) for m_b, k_b in zip(m_list, ks)]
    lens = [m_b + pad - f + 1 for m_b, f in zip(m_list, first)]
    off = _offsets(lens)
    g = _gen(device, seed)
    q, k, v, a, bt = _draw_tokens(g, off[-1], H, d, d, dtype, device, alpha_rng, beta_hi)
    la, lb = [], []
    td = _tdtype(dtype)
    for _ in range(layers - 1):
        lo, hi = alpha_rng
        la.append((lo + (hi - lo) * torch.rand(off[-1], H, generator=g, device=device)).to(td))
        lb.append((beta_hi * torch.rand(off[-1], H, generator=g, device=device)).to(td))
    return Workload(name=name or f"tail_B{B}_H{H}_m{m}_r{r_num}of{r_den}_L{layers}", op="tail",
                    B=B, H=H, dk=d, dv=d, dtype=dtype, flags=NORMALIZE_K | NORMALIZE_Q,
                    q=q, k=k, v=v, alpha=a, beta=bt, tok_offset=off, first_pos=first,
                    n_tokens=[m_b + pad for m_b in m_list], m=m_list, r_num=r_num,
                    r_den=r_den, layers=layers, layer_alpha=la or None,
                    layer_beta=lb or None, seed=seed)


def cluster_keys(w: Workload, n_dirs: int = 4, spread: float = 0.15, seed: int = 0) -> Workload:
    """Replace the keys by unit keys clustered near ``n_dirs`` random directions
    per head: key = (c_j + spread * z) / ||c_j + spread * z|| with a random
    cluster j per token, c_j unit and z ~ N(0, I / d_k).  Inside a cluster the
    cosine between two keys is about 1 / (1 + spread^2), i.e. the Gram matrix
    of a chunk's keys is close to rank n_dirs."""
    g = torch.Generator().manual_seed(10_000 + seed)
    rows, H, dk = w.k.shape
    centres = _unit_rows(torch.randn(H, n_dirs, dk, generator=g, dtype=torch.float64))
    pick = torch.randint(0, n_dirs, (rows, H), generator=g)
    z = torch.randn(rows, H, dk, generator=g, dtype=torch.float64) / dk ** 0.5
    k = _unit_rows(centres[torch.arange(H)[None, :], pick] + spread * z)
    w.k = k.to(dtype=w.k.dtype, device=w.k.device)
    return w


def scale_rows(w: Workload, which: str = "k", log10_range=(-3.0, 3.0), zero_every: int = 0,
               extreme=(), seed: int = 0) -> Workload:
    """Multiply each row of q or k by 10^u, u ~ U(log10_range), set every
    ``zero_every``-th row (if > 0) to zero, and give the rows listed in
    ``extreme`` as (row, factor) that exact factor instead (e.g. 1e-20, 1e20)."""
    g = torch.Generator().manual_seed(20_000 + seed)
    t = getattr(w, which)
    rows, H, _ = t.shape
    f = torch.pow(10.0, torch.empty(rows, H, 1, dtype=torch.float64).uniform_(*log10_range, generator=g))
    if zero_every > 0:
        f[::zero_every] = 0.0
    for r, fac in extreme:
        f[r] = fac
    x = t.to(device="cpu", dtype=torch.float64) * f
    setattr(w, which, x.to(dtype=t.dtype, device=t.device))
    return w


def poison_outside(w: Workload, spans) -> None:
    """Fill every row that lies outside spans[b] = (first position, length) with NaN."""
    keep = torch.zeros(w.rows, dtype=torch.bool)
    for b, (p0, n) in enumerate(spans):
        r0 = w.tok_offset[b] + (p0 - w.first_pos[b])
        keep[r0:r0 + n] = True
    bad = (~keep).to(w.q.device)
    for t in (w.q, w.k, w.v, w.alpha, w.beta):
        t[bad] = float("nan")


# The five headline workloads, at their full sizes, by name.
WORKLOADS = {
    "tiny_prefill_d16": lambda device: tiny_prefill(device=device),
    "resume_B8_H16_N8192": lambda device: resume(device=device),
    "tail5_B16_H32_m32768": lambda device: tail(device=device),
    "tail10_grouped_B16_H32_m32768_L3": lambda device: tail(device=device, seed=4, r_num=10, r_den=100, layers=3,
                                                             name="tail_grouped_B16_H32_m32768_r10_L3"),
    "prefill_emit_B4_H32_N65536": lambda device: prefill(device=device),
}


def named(name: str, device="cpu"):
    """One of the five headline workloads (WORKLOADS) at full size."""
    return WORKLOADS[name](device)
