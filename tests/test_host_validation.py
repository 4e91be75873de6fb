"""Host-side argument validation of the C ABI.

Each call passes placeholder device addresses that validation must reject
before any HIP API is touched.  The module runs only where no GPU is visible,
so that a validation bug can never become a launch on real memory.
"""
import ctypes
import os

import pytest
import torch


@pytest.fixture(scope="module")
def gdn():
    import gated_delta_rule_scan_amd as g
    if not os.path.exists(g.library_path()):
        from gated_delta_rule_scan_amd.build import build
        build()
    return g


# --- argument validation (host only: each call fails before any launch) ------
# These calls pass placeholder device addresses that validation must reject.
# They run only where no GPU is visible, so that a validation bug can never
# turn into a launch on real memory.

FAKE = 0x1000  # never dereferenced: validation rejects the call first
pytestmark = pytest.mark.skipif(torch.cuda.device_count() > 0,
                                reason="placeholder-pointer validation runs only without a GPU")


def _call_tail(gdn, shape_kw=None, **kw):
    lib = gdn.load()
    sk = dict(B=2, H=2, dk=128, dv=128, dtype=1, flags=1)
    sk.update(shape_kw or {})
    sh = gdn._Shape(**sk)
    a = dict(off=[0, 10, 20], first=None, m=[10, 10], r_num=5, r_den=100,
             state=FAKE, o=FAKE)
    a.update(kw)
    off = gdn._i64(a["off"])
    first = gdn._i64(a["first"])
    m = gdn._i64(a["m"])
    p = ctypes.c_void_p(FAKE)
    st = lib.gdn_tail_replay(ctypes.byref(sh), p, p, p, p, p, gdn._p64(off), gdn._p64(first),
                             gdn._p64(m), a["r_num"], a["r_den"],
                             ctypes.c_void_p(a["state"]) if a["state"] else None,
                             ctypes.c_void_p(a["o"]) if a["o"] else None, None, None)
    return st, lib.gdn_last_error().decode()


@pytest.mark.parametrize("shape_kw,code", [
    ({"dk": 96}, 2), ({"dv": 8}, 2), ({"dtype": 7}, 1), ({"H": 0}, 1), ({"B": -1}, 1),
    ({"flags": 1 << 20}, 1), ({"flags": 256 | 512}, 1),
])
def test_shape_errors(gdn, shape_kw, code):
    st, msg = _call_tail(gdn, shape_kw)
    assert st == code and msg


@pytest.mark.parametrize("kw,needle", [
    (dict(off=[0, 10, 5]), "decreases"),
    (dict(off=[-1, 10, 20]), "< 0"),
    (dict(first=[0, 1]), "h_first_pos"),
    (dict(m=[11, 10]), "not stored"),
    (dict(m=[-3, 10]), "h_m"),
    (dict(r_den=0), "ratio"),
    (dict(r_num=-1), "ratio"),
    (dict(state=0), "state_out"),
])
def test_tail_argument_errors(gdn, kw, needle):
    st, msg = _call_tail(gdn, **kw)
    assert st == 1 and needle in msg, msg


@pytest.mark.parametrize("kw,needle", [
    (dict(state=FAKE + (1 << 31)), "o overlaps q, k, v"),                 # o == the inputs
    (dict(state=FAKE, o=FAKE + (1 << 30)), "state buffer overlaps"),      # state_out == the inputs
    (dict(state=FAKE + 8192, o=FAKE + (1 << 30)), "state buffer overlaps"),  # starts inside the span rows
])
def test_outputs_must_not_overlap_inputs(gdn, kw, needle):
    """The kernels write o and the states while they read q, k, v, alpha and
    beta; a call where they share memory is refused before anything is queued."""
    st, msg = _call_tail(gdn, **kw)
    assert st == 1 and needle in msg, msg


def test_tail_span_outside_stored_tail_rows(gdn):
    # rows hold positions 91..100 of each request; m = 100, r = 20% needs 81..100
    st, msg = _call_tail(gdn, first=[91, 91], m=[100, 100], r_num=20, r_den=100)
    assert st == 1 and "not stored" in msg


def test_pointer_alignment(gdn):
    """Inputs must sit at their element size, states at 16 bytes; a chunked
    launch that is required needs 16-byte aligned rows.  All rejected before
    any launch."""
    lib = gdn.load()

    def call(q=FAKE, k=FAKE, alpha=FAKE, state=FAKE, flags=1):
        sh = gdn._Shape(B=2, H=2, dk=128, dv=128, dtype=1, flags=flags)
        off, m = gdn._i64([0, 10, 20]), gdn._i64([10, 10])
        p = ctypes.c_void_p(FAKE)
        st = lib.gdn_tail_replay(ctypes.byref(sh), ctypes.c_void_p(q), ctypes.c_void_p(k), p,
                                 ctypes.c_void_p(alpha), p, gdn._p64(off), None, gdn._p64(m), 5, 100,
                                 ctypes.c_void_p(state), p, None, None)
        return st, lib.gdn_last_error().decode()

    st, msg = call(q=FAKE + 1)
    assert st == 1 and "element size" in msg
    st, msg = call(alpha=FAKE + 3)
    assert st == 1 and "element size" in msg
    st, msg = call(state=FAKE + 8)
    assert st == 1 and "16-byte" in msg
    # bf16 rows two bytes off: fine for the per-token kernel, refused when the
    # chunked kernel is required
    st, msg = call(k=FAKE + 2, flags=1 | 512)
    assert st == 2 and "16-byte" in msg


def test_chunked_required_but_unavailable_for_f32(gdn):
    st, msg = _call_tail(gdn, {"dtype": 0, "flags": 512})
    assert st == 2 and "CHUNKED" in msg


def _call_resume(gdn, pos, depth, states=FAKE, out=FAKE, M=None, off=(0, 50)):
    lib = gdn.load()
    B = len(depth)
    sh = gdn._Shape(B, 1, 16, 16, 0, 1)
    offa = gdn._i64(off)
    posa = gdn._i64(pos)
    M = len(pos) // B if M is None else M
    p = ctypes.c_void_p(FAKE)
    st = lib.gdn_resume(ctypes.byref(sh), p, p, p, p, p, gdn._p64(offa), None, gdn._p64(posa), M,
                        ctypes.c_void_p(states) if states else None, gdn._p64(gdn._i64(depth)),
                        ctypes.c_void_p(out) if out else None, None, None, None)
    return st, lib.gdn_last_error().decode()


def test_resume_errors(gdn):
    assert _call_resume(gdn, [5, 5], [7])[0] == 1          # not strictly increasing
    assert _call_resume(gdn, [0, 5], [7])[0] == 1          # position < 1
    assert _call_resume(gdn, [5, 9], [-1])[0] == 1         # negative depth
    assert _call_resume(gdn, [5, 9], [60])[0] == 1         # span beyond stored rows
    assert _call_resume(gdn, [5, 9], [7], states=0)[0] == 1  # selects a slot, no store
    st, msg = _call_resume(gdn, [5] * 1, [7], M=300)
    assert st == 2 and "exceeds" in msg
    # state_out overlapping another request's selected slot is rejected
    base = 0x100000
    slot = 16 * 16 * 4
    # request 1 reads slot (1, 1) = bytes [3 slot, 4 slot); request 0 writes there
    st, msg = _call_resume(gdn, [5, 9, 5, 9], [7, 9], states=base, out=base + 3 * slot,
                           off=(0, 50, 100))
    assert st == 1 and "overlaps" in msg


def test_prefill_errors(gdn):
    lib = gdn.load()
    sh = gdn._Shape(1, 1, 16, 16, 0, 1)
    p = ctypes.c_void_p(FAKE)
    off = gdn._i64([0, 20])

    store = FAKE + (1 << 20)

    def call(pos, first=None, states=store, out=FAKE + 10 ** 9):
        posa = gdn._i64(pos)
        st = lib.gdn_prefill_emit_checkpoints(
            ctypes.byref(sh), p, p, p, p, p, gdn._p64(off), gdn._p64(gdn._i64(first)),
            gdn._p64(posa), len(pos), ctypes.c_void_p(states) if states else None,
            ctypes.c_void_p(out), None, None)
        return st, lib.gdn_last_error().decode()

    def fails(needle, *a, **kw):
        st, msg = call(*a, **kw)
        return st == 1 and needle in msg

    assert fails("", [5, 21])                  # beyond N
    assert fails("increasing", [5, 4])         # not increasing
    assert fails("", [5], first=[2])           # prefill needs position 1
    assert fails("", [5], states=0)            # emission store missing
    assert fails("overlap", [5], out=store)    # state_out overlaps the store
    # the emission store is written while the input rows are read (20 rows x 16 fp32 = 1280 B)
    assert fails("ckpt_states overlaps", [5], states=FAKE + 1024)


def test_split_prefill_workspace_checks(gdn):
    lib = gdn.load()
    sh = gdn._Shape(B=1, H=2, dk=128, dv=128, dtype=1, flags=1)
    need = lib.gdn_prefill_split_workspace_bytes(ctypes.byref(sh))
    assert need == 4 * 1 * 2 * 128 * 128 * 4
    off = (ctypes.c_int64 * 2)(0, 1000)
    pos = (ctypes.c_int64 * 1)(500)

    def call(ws, nbytes, shape=sh, state=FAKE):
        return lib.gdn_prefill_emit_checkpoints_split(
            ctypes.byref(shape), FAKE, FAKE, FAKE, FAKE, FAKE, off, None, pos, 1, 0x200000000,
            state, FAKE, ws, nbytes, None)

    assert call(None, need) == 1
    assert call(0x900000000, need - 1) == 1
    assert call(0x900000008, need) == 1 and b"16-byte" in lib.gdn_last_error()
    # the workspace may not overlap the final states
    assert call(0x900000000, need, state=0x900000000 + 4096) == 1
    assert b"overlaps" in lib.gdn_last_error()
    sh2 = gdn._Shape(B=1, H=2, dk=128, dv=64, dtype=1, flags=0)
    assert call(0x900000000, 10 ** 9, shape=sh2) == 2


def test_overlapped_replay_argument_errors(gdn):
    """The transfer arguments are checked before anything is queued."""
    lib = gdn.load()
    sh = gdn._Shape(B=2, H=2, dk=128, dv=128, dtype=1, flags=1)
    off = gdn._i64([0, 10, 20])
    m = gdn._i64([10, 10])
    p = ctypes.c_void_p(FAKE)

    def call(dst, src, nbytes, event, r_den=100):
        return lib.gdn_tail_replay_with_h2d(ctypes.byref(sh), p, p, p, p, p, gdn._p64(off), None, gdn._p64(m),
                                            5, r_den, p, p, None, dst, src, nbytes, None, None, event)

    assert call(FAKE, FAKE, 1024, None) == 1 and "copy_done" in lib.gdn_last_error().decode()
    assert call(None, FAKE, 1024, FAKE) == 1 and "kv_dst" in lib.gdn_last_error().decode()
    assert call(FAKE, None, 1024, FAKE) == 1
    # replay arguments are validated first: nothing is queued on an invalid ratio
    assert call(FAKE, FAKE, 1024, FAKE, r_den=0) == 1 and "ratio" in lib.gdn_last_error().decode()


@pytest.mark.parametrize("case", ["misaligned q, chunked required", "NULL k", "o without q",
                                  "state_out misaligned"])
def test_overlapped_replay_checks_the_replay_before_the_copy(gdn, case):
    """Every argument of the replay (pointers, alignment, kernel choice) is
    checked before the copy is queued: with placeholder copy arguments, a
    queued copy would fail in the runtime (GDN_ERR_HIP, no GPU here), so the
    replay's own error code shows that nothing was queued."""
    lib = gdn.load()
    flags = 1 | (512 if case.startswith("misaligned q") else 0)
    sh = gdn._Shape(B=2, H=2, dk=128, dv=128, dtype=1, flags=flags)
    off = gdn._i64([0, 10, 20])
    m = gdn._i64([10, 10])
    p = ctypes.c_void_p(FAKE)
    q, k, state, o = p, p, p, p
    if case.startswith("misaligned q"):
        q = ctypes.c_void_p(FAKE + 2)
    elif case == "NULL k":
        k = None
    elif case == "o without q":
        q = None
    else:
        state = ctypes.c_void_p(FAKE + 4)
    st = lib.gdn_tail_replay_with_h2d(ctypes.byref(sh), q, k, p, p, p, gdn._p64(off), None, gdn._p64(m),
                                      5, 100, state, o, None, p, p, 1 << 20, None, None, p)
    want = 2 if case.startswith("misaligned q") else 1
    assert st == want, (st, lib.gdn_last_error().decode())


def test_noalloc_split_prefill_rejects_sizes_beyond_its_scratch(gdn):
    """The allocation-free split prefill refuses a shape whose workspace
    (4 B H d_v d_k floats) exceeds its fixed scratch, before any HIP call."""
    lib = gdn.load()
    assert gdn.SPLIT_SCRATCH_BYTES == 32 << 20
    p = ctypes.c_void_p(FAKE)
    ck, st = ctypes.c_void_p(1 << 36), ctypes.c_void_p(1 << 40)  # disjoint placeholder outputs
    n = 1000

    def call(B, H, d, M=1):
        sh = gdn._Shape(B=B, H=H, dk=d, dv=d, dtype=1, flags=1)
        off = gdn._i64([n * b for b in range(B + 1)])
        pos = gdn._i64([n] * (B * M))
        return lib.gdn_prefill_emit_checkpoints_split_noalloc(ctypes.byref(sh), p, p, p, p, p, gdn._p64(off),
                                                              None, gdn._p64(pos), M, ck, st, p, None)

    # 4 x 33 x 128 x 128 x 16 bytes = 33 MiB > 32 MiB
    assert call(4, 33, 128) == 2 and "scratch" in lib.gdn_last_error().decode()
    assert call(1, 129, 128) == 2
    # d_k != d_v, and a bad checkpoint list, are refused like the split prefill's
    sh = gdn._Shape(B=1, H=1, dk=64, dv=128, dtype=1, flags=1)
    off = gdn._i64([0, n])
    pos = gdn._i64([n])
    assert lib.gdn_prefill_emit_checkpoints_split_noalloc(ctypes.byref(sh), p, p, p, p, p, gdn._p64(off), None,
                                                          gdn._p64(pos), 1, ck, st, p, None) == 2
    sh = gdn._Shape(B=1, H=1, dk=128, dv=128, dtype=1, flags=1)
    bad = gdn._i64([n + 1])
    assert lib.gdn_prefill_emit_checkpoints_split_noalloc(ctypes.byref(sh), p, p, p, p, p, gdn._p64(off), None,
                                                          gdn._p64(bad), 1, ck, st, p, None) == 1


def _call_group(gdn, L=3, shape_kw=None, alphas=None, betas=None, state=FAKE + (1 << 31), o=FAKE + (1 << 30),
                arrays=True):
    lib = gdn.load()
    sk = dict(B=2, H=2, dk=128, dv=128, dtype=1, flags=1)
    sk.update(shape_kw or {})
    sh = gdn._Shape(**sk)
    off, m = gdn._i64([0, 10, 20]), gdn._i64([10, 10])
    n = max(L, 1)
    pa = (ctypes.c_void_p * n)(*(alphas if alphas is not None else [FAKE] * n))
    pb = (ctypes.c_void_p * n)(*(betas if betas is not None else [FAKE] * n))
    p = ctypes.c_void_p(FAKE)
    st = lib.gdn_tail_replay_group(ctypes.byref(sh), L, p, p, p, pa if arrays else None, pb if arrays else None,
                                   gdn._p64(off), None, gdn._p64(m), 5, 100,
                                   ctypes.c_void_p(state) if state else None, ctypes.c_void_p(o) if o else None,
                                   None, None)
    return st, lib.gdn_last_error().decode()


@pytest.mark.parametrize("kw,code,needle", [
    (dict(L=0), 1, "L = 0"),
    (dict(L=5), 1, "L = 5"),
    (dict(arrays=False), 1, "alpha and beta"),
    (dict(shape_kw={"dv": 64}), 2, "d_k = d_v"),
    (dict(o=0), 1, "o is NULL"),
    (dict(state=0), 1, "state_out is NULL"),
    (dict(o=FAKE + (1 << 31)), 1, "o and state_out overlap"),
    (dict(o=FAKE), 1, "o overlaps q, k, v"),
    (dict(state=FAKE), 1, "state buffer overlaps"),
    (dict(alphas=[FAKE, FAKE, None]), 1, "non-NULL"),
    (dict(betas=[FAKE, FAKE + 1, FAKE]), 1, "aligned"),
])
def test_group_argument_errors(gdn, kw, code, needle):
    """Every layer's arguments are checked before any launch."""
    st, msg = _call_group(gdn, **kw)
    assert st == code and needle in msg, (st, msg)
