"""Python binding of libgdnreplay (Gated DeltaNet span replay on MI355X).

Argument marshalling only: every step of the replay runs in the HIP kernels of
``libgdnreplay.so`` behind the C ABI of ``include/gdnreplay.h``.  PyTorch
supplies device memory and the current stream.  There is no fallback: if the
shared library is missing or cannot be loaded, every call raises.

Layout (see the header for the full contract):
  q, k [rows, H, d_k], v [rows, H, d_v], alpha, beta [rows, H]  (float32 or bfloat16)
  request b owns rows tok_offset[b]..tok_offset[b+1]-1, whose first row holds
  the token at 1-based position first_pos[b].
  States are float32 [B, H, d_v, d_k]; checkpoint stores [B, M, H, d_v, d_k].
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import numpy as np
import torch

__all__ = [
    "GDNError", "NORMALIZE_K", "NORMALIZE_Q", "KERNEL_RECURRENT", "KERNEL_CHUNKED",
    "MAX_CHECKPOINTS", "library_path", "load", "version", "kernel_for", "tail_len", "select_checkpoint",
    "tail_replay", "tail_replay_with_h2d", "resume", "prefill_emit_checkpoints",
    "prefill_split_workspace_bytes", "prefill_emit_checkpoints_split", "SPLIT_SCRATCH_BYTES",
    "prefill_emit_checkpoints_split_noalloc",
    "expected_recompute", "balanced_checkpoints", "plan_checkpoints",
]

NORMALIZE_K = 1
NORMALIZE_Q = 2
KERNEL_RECURRENT = 256
KERNEL_CHUNKED = 512
MAX_CHECKPOINTS = 192
SPLIT_SCRATCH_BYTES = 32 << 20  # GDN_SPLIT_SCRATCH_BYTES

_DTYPES = {torch.float32: 0, torch.bfloat16: 1}
_STATUS = {0: "GDN_OK", 1: "GDN_ERR_INVALID_ARGUMENT", 2: "GDN_ERR_UNSUPPORTED", 3: "GDN_ERR_HIP"}

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libgdnreplay.so")
_lib = None


class GDNError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{_STATUS.get(status, status)}: {message}")
        self.status = status


class _Shape(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("H", ctypes.c_int32), ("dk", ctypes.c_int32),
                ("dv", ctypes.c_int32), ("dtype", ctypes.c_int32), ("flags", ctypes.c_uint32)]


def library_path() -> str:
    return _LIB_PATH


def load():
    """Load libgdnreplay.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(
            f"{_LIB_PATH} is missing: build it with gated_delta_rule_scan_amd.build.build() "
            "(or __graft_entry__.build()); there is no fallback path")
    lib = ctypes.CDLL(_LIB_PATH)
    vp, i64p, i32p = ctypes.c_void_p, ctypes.POINTER(ctypes.c_int64), ctypes.POINTER(ctypes.c_int32)
    shp = ctypes.POINTER(_Shape)
    lib.gdn_version.restype = ctypes.c_char_p
    lib.gdn_last_error.restype = ctypes.c_char_p
    lib.gdn_kernel_for.argtypes = [shp]
    lib.gdn_kernel_for.restype = ctypes.c_int32
    lib.gdn_tail_len.argtypes = [ctypes.c_int64] * 3
    lib.gdn_tail_len.restype = ctypes.c_int64
    lib.gdn_select_checkpoint.argtypes = [i64p, ctypes.c_int32, ctypes.c_int64]
    lib.gdn_select_checkpoint.restype = ctypes.c_int32
    lib.gdn_tail_replay.argtypes = [shp, vp, vp, vp, vp, vp, i64p, i64p, i64p, ctypes.c_int64,
                                    ctypes.c_int64, vp, vp, i64p, vp]
    lib.gdn_tail_replay.restype = ctypes.c_int
    lib.gdn_tail_replay_group.argtypes = [shp, ctypes.c_int32, vp, vp, vp, ctypes.POINTER(vp),
                                          ctypes.POINTER(vp), i64p, i64p, i64p, ctypes.c_int64,
                                          ctypes.c_int64, vp, vp, i64p, vp]
    lib.gdn_tail_replay_group.restype = ctypes.c_int
    lib.gdn_tail_replay_with_h2d.argtypes = [shp, vp, vp, vp, vp, vp, i64p, i64p, i64p, ctypes.c_int64,
                                             ctypes.c_int64, vp, vp, i64p, vp, vp, ctypes.c_size_t,
                                             vp, vp, vp]
    lib.gdn_tail_replay_with_h2d.restype = ctypes.c_int
    lib.gdn_resume.argtypes = [shp, vp, vp, vp, vp, vp, i64p, i64p, i64p, ctypes.c_int32, vp,
                               i64p, vp, vp, i32p, vp]
    lib.gdn_resume.restype = ctypes.c_int
    lib.gdn_prefill_emit_checkpoints.argtypes = [shp, vp, vp, vp, vp, vp, i64p, i64p, i64p,
                                                 ctypes.c_int32, vp, vp, vp, vp]
    lib.gdn_prefill_emit_checkpoints.restype = ctypes.c_int
    lib.gdn_prefill_split_workspace_bytes.argtypes = [shp]
    lib.gdn_prefill_split_workspace_bytes.restype = ctypes.c_size_t
    lib.gdn_prefill_emit_checkpoints_split.argtypes = [shp, vp, vp, vp, vp, vp, i64p, i64p, i64p,
                                                       ctypes.c_int32, vp, vp, vp, vp, ctypes.c_size_t, vp]
    lib.gdn_prefill_emit_checkpoints_split.restype = ctypes.c_int
    lib.gdn_prefill_emit_checkpoints_split_noalloc.argtypes = [shp, vp, vp, vp, vp, vp, i64p, i64p, i64p,
                                                               ctypes.c_int32, vp, vp, vp, vp]
    lib.gdn_prefill_emit_checkpoints_split_noalloc.restype = ctypes.c_int
    f64p = ctypes.POINTER(ctypes.c_double)
    lib.gdn_expected_recompute.argtypes = [f64p, ctypes.c_int64, i64p, ctypes.c_int32]
    lib.gdn_expected_recompute.restype = ctypes.c_double
    lib.gdn_balanced_checkpoints.argtypes = [ctypes.c_int64, ctypes.c_int32, i64p]
    lib.gdn_balanced_checkpoints.restype = ctypes.c_int32
    lib.gdn_plan_checkpoints.argtypes = [f64p, ctypes.c_int64, ctypes.c_int32, i64p, f64p]
    lib.gdn_plan_checkpoints.restype = ctypes.c_int
    _lib = lib
    return lib


def version() -> str:
    return load().gdn_version().decode()


def _i64(seq) -> Optional[np.ndarray]:
    if seq is None:
        return None
    return np.ascontiguousarray(np.asarray(seq, dtype=np.int64).reshape(-1))


def _p64(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.POINTER(ctypes.c_int64))


def kernel_for(B: int, H: int, dk: int, dv: int, dtype: torch.dtype, flags: int = 0) -> str:
    """Name of the kernel the library runs for this shape: "recurrent" or "chunked"."""
    sh = _shape(B, H, dk, dv, _DTYPES[dtype], flags)
    r = int(load().gdn_kernel_for(ctypes.byref(sh)))
    if r < 0:
        raise GDNError(2, f"no kernel for B={B} H={H} d_k={dk} d_v={dv} {dtype} flags={flags}")
    return "chunked" if r == 1 else "recurrent"


def tail_len(m: int, r_num: int, r_den: int) -> int:
    """k = ceil(r m), exact, capped at m; -1 for invalid arguments."""
    return int(load().gdn_tail_len(int(m), int(r_num), int(r_den)))


def select_checkpoint(positions: Sequence[int], depth: int) -> int:
    """1-based index of the deepest checkpoint <= depth (0: none); -1 if invalid."""
    pos = _i64(positions)
    return int(load().gdn_select_checkpoint(_p64(pos), int(pos.size), int(depth)))


def _f64(seq) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(seq, dtype=np.float64).reshape(-1))


def expected_recompute(p: Sequence[float], positions: Sequence[int]) -> float:
    """R(p, C): expected recomputed tokens for depth weights p[0..N] and the
    checkpoint positions (host computation in the library); -1.0 if invalid."""
    pa, pos = _f64(p), _i64(positions)
    return float(load().gdn_expected_recompute(pa.ctypes.data_as(ctypes.POINTER(ctypes.c_double)),
                                               pa.size - 1, _p64(pos), int(pos.size)))


def balanced_checkpoints(N: int, M: int) -> np.ndarray:
    """M positions floor(i (N+1) / (M+1)): gaps that differ by at most one."""
    out = np.zeros(max(int(M), 0), dtype=np.int64)
    if int(load().gdn_balanced_checkpoints(int(N), int(M), _p64(out))) != 0:
        raise GDNError(1, f"invalid balanced placement N={N} M={M}")
    return out


def plan_checkpoints(p: Sequence[float], M: int):
    """Optimal M positions for depth weights p[0..N] (O(N M) dynamic programme).
    Returns (positions int64 [M], minimal expected recomputation)."""
    pa = _f64(p)
    out = np.zeros(max(int(M), 0), dtype=np.int64)
    cost = ctypes.c_double(0.0)
    _check(load().gdn_plan_checkpoints(pa.ctypes.data_as(ctypes.POINTER(ctypes.c_double)), pa.size - 1,
                                       int(M), _p64(out), ctypes.byref(cost)))
    return out, float(cost.value)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _check_tensors(q, k, v, alpha, beta, o):
    dt = k.dtype
    if dt not in _DTYPES:
        raise TypeError(f"unsupported element type {dt}; use float32 or bfloat16")
    for name, t in (("q", q), ("k", k), ("v", v), ("alpha", alpha), ("beta", beta), ("o", o)):
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError(f"{name} must be a device tensor")
        if t.device != k.device:
            raise ValueError(f"{name} is on {t.device}, k on {k.device}: one device per call")
        if t.dtype != dt:
            raise TypeError(f"{name} has dtype {t.dtype}, expected {dt}")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    rows, H, dk = k.shape
    dv = v.shape[2]
    if v.shape[:2] != (rows, H) or alpha.shape != (rows, H) or beta.shape != (rows, H):
        raise ValueError("v, alpha, beta must match k's [rows, H] layout")
    if q is not None and q.shape != k.shape:
        raise ValueError("q must have k's shape")
    if o is not None and o.shape != v.shape:
        raise ValueError("o must have v's shape")
    return rows, H, dk, dv, _DTYPES[dt]


def _shape(B, H, dk, dv, dtype, flags):
    return _Shape(int(B), int(H), int(dk), int(dv), int(dtype), int(flags))


def _state(t: Optional[torch.Tensor], shape, device, name):
    if t is None:
        return torch.empty(shape, dtype=torch.float32, device=device)
    if t.dtype != torch.float32 or not t.is_contiguous() or tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must be contiguous float32 of shape {tuple(shape)}")
    if not t.is_cuda or t.device != device:
        raise ValueError(f"{name} must be a device tensor on {device}")
    return t


def _check(status: int):
    if status != 0:
        raise GDNError(status, load().gdn_last_error().decode())


def _rows_meta(tok_offset, first_pos, rows, B):
    off = _i64(tok_offset)
    if off.size != B + 1:
        raise ValueError("tok_offset must have B + 1 entries")
    if off[-1] > rows:
        raise ValueError(f"tok_offset[-1] = {off[-1]} exceeds the {rows} stored rows")
    fp = _i64(first_pos)
    if fp is not None and fp.size != B:
        raise ValueError("first_pos must have B entries")
    return off, fp


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _call(device, fn, *args):
    """Run a library entry point with `device` current (the library reads the
    current device's properties and its scratch array on that device)."""
    with torch.cuda.device(device):
        _check(fn(*args))


def tail_replay(q, k, v, alpha, beta, tok_offset, m, r_num, r_den, *, first_pos=None,
                flags=NORMALIZE_K, state_out=None, o=None, want_o=True):
    """Zero-start replay of the last ceil(r m_b) positions of each request.

    Returns (state_out [B,H,d_v,d_k] float32, o or None, k_b list)."""
    if want_o and o is None:
        o = torch.empty_like(v)
    rows, H, dk, dv, dt = _check_tensors(q if o is not None else None, k, v, alpha, beta, o)
    mm = _i64(m)
    B = int(mm.size)
    off, fp = _rows_meta(tok_offset, first_pos, rows, B)
    state_out = _state(state_out, (B, H, dv, dk), k.device, "state_out")
    kout = np.zeros(B, np.int64)
    sh = _shape(B, H, dk, dv, dt, flags)
    _call(k.device, load().gdn_tail_replay,
        ctypes.byref(sh), _ptr(q if o is not None else None), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta),
        _p64(off), _p64(fp), _p64(mm), int(r_num), int(r_den), _ptr(state_out), _ptr(o), _p64(kout),
        _stream(k.device))
    return state_out, o, [int(x) for x in kout]


def tail_replay_group(q, k, v, alphas, betas, tok_offset, m, r_num, r_den, *, first_pos=None,
                      flags=NORMALIZE_K, state_out=None, o=None):
    """Tail replay of a group of len(alphas) layers chained by identity mixing
    (layer l + 1's q = k = v is layer l's output), the same span on every layer.

    Returns (state_out [L,B,H,d_v,d_k] float32, o [L,rows,H,d_v], k_b list)."""
    L = len(alphas)
    if len(betas) != L:
        raise ValueError("one beta per alpha")
    rows, H, dk, dv, dt = _check_tensors(q, k, v, alphas[0], betas[0], None)
    for a_, b_ in zip(alphas, betas):
        _check_tensors(None, k, v, a_, b_, None)
    if o is None:
        o = torch.empty((L,) + tuple(v.shape), dtype=v.dtype, device=v.device)
    if tuple(o.shape) != (L,) + tuple(v.shape) or o.dtype != v.dtype or not o.is_contiguous():
        raise ValueError("o must be a contiguous [L, rows, H, d_v] tensor of v's dtype")
    if not o.is_cuda or o.device != k.device:
        raise ValueError(f"o must be a device tensor on {k.device}")
    mm = _i64(m)
    B = int(mm.size)
    off, fp = _rows_meta(tok_offset, first_pos, rows, B)
    state_out = _state(state_out, (L, B, H, dv, dk), k.device, "state_out")
    kout = np.zeros(B, np.int64)
    sh = _shape(B, H, dk, dv, dt, flags)
    pa = (ctypes.c_void_p * L)(*[_ptr(x) for x in alphas])
    pb = (ctypes.c_void_p * L)(*[_ptr(x) for x in betas])
    _call(k.device, load().gdn_tail_replay_group,
        ctypes.byref(sh), L, _ptr(q), _ptr(k), _ptr(v), pa, pb, _p64(off), _p64(fp), _p64(mm), int(r_num),
        int(r_den), _ptr(state_out), _ptr(o), _p64(kout), _stream(k.device))
    return state_out, o, [int(x) for x in kout]


def tail_replay_with_h2d(q, k, v, alpha, beta, tok_offset, m, r_num, r_den, kv_src, kv_dst,
                         copy_stream, copy_done, *, first_pos=None, flags=NORMALIZE_K,
                         state_out=None, o=None, want_o=True):
    """tail_replay on the current stream, overlapped with a host-to-device copy of
    kv_src (pinned CPU tensor) into kv_dst (device tensor of the same byte size)
    on copy_stream; the current stream waits for the copy (copy_done, a
    torch.cuda.Event) before any later work.  Returns what tail_replay returns."""
    if want_o and o is None:
        o = torch.empty_like(v)
    rows, H, dk, dv, dt = _check_tensors(q if o is not None else None, k, v, alpha, beta, o)
    nbytes = kv_src.numel() * kv_src.element_size()
    if kv_src.is_cuda or not kv_dst.is_cuda or not kv_src.is_contiguous() or not kv_dst.is_contiguous():
        raise ValueError("kv_src must be a contiguous host tensor and kv_dst a contiguous device tensor")
    if kv_dst.numel() * kv_dst.element_size() != nbytes:
        raise ValueError("kv_src and kv_dst differ in byte size")
    if not copy_done.cuda_event:
        copy_done.record(copy_stream)  # torch creates the event on its first record
    mm = _i64(m)
    B = int(mm.size)
    off, fp = _rows_meta(tok_offset, first_pos, rows, B)
    state_out = _state(state_out, (B, H, dv, dk), k.device, "state_out")
    kout = np.zeros(B, np.int64)
    sh = _shape(B, H, dk, dv, dt, flags)
    _call(k.device, load().gdn_tail_replay_with_h2d,
        ctypes.byref(sh), _ptr(q if o is not None else None), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta),
        _p64(off), _p64(fp), _p64(mm), int(r_num), int(r_den), _ptr(state_out), _ptr(o), _p64(kout),
        ctypes.c_void_p(kv_dst.data_ptr()), ctypes.c_void_p(kv_src.data_ptr()), nbytes,
        _stream(k.device), ctypes.c_void_p(copy_stream.cuda_stream), ctypes.c_void_p(copy_done.cuda_event))
    return state_out, o, [int(x) for x in kout]


def resume(q, k, v, alpha, beta, tok_offset, ckpt_pos, ckpt_states, depth, *, first_pos=None,
           flags=NORMALIZE_K, state_out=None, o=None, want_o=True):
    """Resume each request from its deepest checkpoint <= depth_b and recompute
    up to depth_b.  ckpt_pos is [B][M]; ckpt_states [B, M, H, d_v, d_k] float32.

    Returns (state_out, o or None, j_b list)."""
    if want_o and o is None:
        o = torch.empty_like(v)
    rows, H, dk, dv, dt = _check_tensors(q if o is not None else None, k, v, alpha, beta, o)
    dd = _i64(depth)
    B = int(dd.size)
    pos = np.ascontiguousarray(np.asarray(ckpt_pos, dtype=np.int64).reshape(B, -1))
    M = int(pos.shape[1])
    off, fp = _rows_meta(tok_offset, first_pos, rows, B)
    if ckpt_states is not None:
        if ckpt_states.dtype != torch.float32 or not ckpt_states.is_contiguous() or \
                tuple(ckpt_states.shape) != (B, M, H, dv, dk):
            raise ValueError(f"ckpt_states must be contiguous float32 [{B},{M},{H},{dv},{dk}]")
        if not ckpt_states.is_cuda or ckpt_states.device != k.device:
            raise ValueError(f"ckpt_states must be a device tensor on {k.device}")
    state_out = _state(state_out, (B, H, dv, dk), k.device, "state_out")
    jout = np.zeros(B, np.int32)
    sh = _shape(B, H, dk, dv, dt, flags)
    _call(k.device, load().gdn_resume,
          ctypes.byref(sh), _ptr(q if o is not None else None), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta),
        _p64(off), _p64(fp), _p64(pos.reshape(-1)), M, _ptr(ckpt_states), _p64(dd), _ptr(state_out), _ptr(o),
        jout.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), _stream(k.device))
    return state_out, o, [int(x) for x in jout]


def prefill_emit_checkpoints(q, k, v, alpha, beta, tok_offset, ckpt_pos, *, flags=NORMALIZE_K,
                             ckpt_states=None, state_out=None, o=None, want_o=True):
    """Full prefill of every request from zero, storing the state after each
    position in ckpt_pos[b] (strictly increasing, in [1, N_b]).

    Returns (ckpt_states [B,M,H,d_v,d_k], state_out [B,H,d_v,d_k], o or None)."""
    if want_o and o is None:
        o = torch.empty_like(v)
    rows, H, dk, dv, dt = _check_tensors(q if o is not None else None, k, v, alpha, beta, o)
    off = _i64(tok_offset)
    B = int(off.size) - 1
    off, _ = _rows_meta(off, None, rows, B)
    pos = np.ascontiguousarray(np.asarray(ckpt_pos, dtype=np.int64).reshape(B, -1))
    M = int(pos.shape[1])
    ckpt_states = _state(ckpt_states, (B, M, H, dv, dk), k.device, "ckpt_states")
    state_out = _state(state_out, (B, H, dv, dk), k.device, "state_out")
    sh = _shape(B, H, dk, dv, dt, flags)
    _call(k.device, load().gdn_prefill_emit_checkpoints,
        ctypes.byref(sh), _ptr(q if o is not None else None), _ptr(k), _ptr(v), _ptr(alpha),
        _ptr(beta), _p64(off), None, _p64(pos.reshape(-1)), M,
        _ptr(ckpt_states) if M > 0 else None, _ptr(state_out), _ptr(o), _stream(k.device))
    return ckpt_states, state_out, o


def prefill_split_workspace_bytes(B: int, H: int, dk: int, dv: int, dtype: torch.dtype = torch.bfloat16) -> int:
    """Device bytes the split prefill needs as workspace."""
    sh = _shape(B, H, dk, dv, _DTYPES[dtype], 0)
    return int(load().gdn_prefill_split_workspace_bytes(ctypes.byref(sh)))


def prefill_emit_checkpoints_split(q, k, v, alpha, beta, tok_offset, ckpt_pos, *, flags=NORMALIZE_K,
                                   ckpt_states=None, state_out=None, o=None, want_o=True, workspace=None):
    """prefill_emit_checkpoints with each long span cut into three segments
    (see the C header); workspace: a device uint8 tensor of at least
    prefill_split_workspace_bytes(...) bytes (allocated here when None).

    Returns (ckpt_states [B,M,H,d_v,d_k], state_out [B,H,d_v,d_k], o or None)."""
    if want_o and o is None:
        o = torch.empty_like(v)
    rows, H, dk, dv, dt = _check_tensors(q if o is not None else None, k, v, alpha, beta, o)
    off = _i64(tok_offset)
    B = int(off.size) - 1
    off, _ = _rows_meta(off, None, rows, B)
    pos = np.ascontiguousarray(np.asarray(ckpt_pos, dtype=np.int64).reshape(B, -1))
    M = int(pos.shape[1])
    ckpt_states = _state(ckpt_states, (B, M, H, dv, dk), k.device, "ckpt_states")
    state_out = _state(state_out, (B, H, dv, dk), k.device, "state_out")
    sh = _shape(B, H, dk, dv, dt, flags)
    need = int(load().gdn_prefill_split_workspace_bytes(ctypes.byref(sh)))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=k.device)
    if not workspace.is_cuda or not workspace.is_contiguous() or workspace.device != k.device:
        raise ValueError(f"workspace must be a contiguous device tensor on {k.device}")
    _call(k.device, load().gdn_prefill_emit_checkpoints_split,
        ctypes.byref(sh), _ptr(q if o is not None else None), _ptr(k), _ptr(v), _ptr(alpha),
        _ptr(beta), _p64(off), None, _p64(pos.reshape(-1)), M,
        _ptr(ckpt_states) if M > 0 else None, _ptr(state_out), _ptr(o),
        _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(k.device))
    return ckpt_states, state_out, o


def prefill_emit_checkpoints_split_noalloc(q, k, v, alpha, beta, tok_offset, ckpt_pos, *, flags=NORMALIZE_K,
                                           ckpt_states=None, state_out=None, o=None, want_o=True):
    """prefill_emit_checkpoints_split with its workspace in the library's fixed
    per-GPU scratch (SPLIT_SCRATCH_BYTES): the library allocates nothing.  The
    caller passes (or this wrapper allocates) only the outputs.  Calls that
    overlap on one GPU share that scratch and must be ordered (one stream).

    Returns (ckpt_states [B,M,H,d_v,d_k], state_out [B,H,d_v,d_k], o or None)."""
    if want_o and o is None:
        o = torch.empty_like(v)
    rows, H, dk, dv, dt = _check_tensors(q if o is not None else None, k, v, alpha, beta, o)
    off = _i64(tok_offset)
    B = int(off.size) - 1
    off, _ = _rows_meta(off, None, rows, B)
    pos = np.ascontiguousarray(np.asarray(ckpt_pos, dtype=np.int64).reshape(B, -1))
    M = int(pos.shape[1])
    ckpt_states = _state(ckpt_states, (B, M, H, dv, dk), k.device, "ckpt_states")
    state_out = _state(state_out, (B, H, dv, dk), k.device, "state_out")
    sh = _shape(B, H, dk, dv, dt, flags)
    _call(k.device, load().gdn_prefill_emit_checkpoints_split_noalloc,
        ctypes.byref(sh), _ptr(q if o is not None else None), _ptr(k), _ptr(v), _ptr(alpha),
        _ptr(beta), _p64(off), None, _p64(pos.reshape(-1)), M,
        _ptr(ckpt_states) if M > 0 else None, _ptr(state_out), _ptr(o), _stream(k.device))
    return ckpt_states, state_out, o
