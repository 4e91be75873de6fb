"""The allocation-free split prefill (gdn_prefill_emit_checkpoints_split_noalloc)
against the split prefill with a caller workspace, through the C ABI: two calls
in a row on one GPU, the second with a smaller input (the fixed scratch then
holds the first call's leftovers), each bit for bit equal to the workspace
path and within the bf16 bar of the fp64 oracle on every pair."""
import pytest
import torch

import workloads as W
import parity as PT

pytestmark = pytest.mark.gpu


def _log(msg):
    print(msg, flush=True)


@pytest.fixture(scope="module")
def gdn():
    import gated_delta_rule_scan_amd as g
    g.load()
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    return g


def _prefill(seed, B, H, lengths, M):
    w = W.prefill(seed=seed, B=B, H=H, d=128, N=max(lengths), M=M, lengths=lengths)
    return PT.to_device(w)


def test_noalloc_split_prefill_matches_the_workspace_path(gdn):
    cases = [
        # the largest input the scratch holds: 4 x 32 pairs, d = 128 (32 MiB of workspace)
        _prefill(301, 4, 32, [3000, 2400, 1900, 800], 5),
        # then a smaller one, over the first call's leftovers
        _prefill(302, 2, 8, [2000, 700], 4),
    ]
    assert gdn.prefill_split_workspace_bytes(4, 32, 128, 128) == gdn.SPLIT_SCRATCH_BYTES
    # the first call in a process loads the library's code object that holds the
    # scratch array (once per GPU); the calls measured below come after it
    w = cases[1]
    gdn.prefill_emit_checkpoints_split_noalloc(w.q, w.k, w.v, w.alpha, w.beta, w.tok_offset, w.ckpt_pos,
                                               flags=w.flags)
    torch.cuda.synchronize()
    for i, w in enumerate(cases):
        _log(f"[no-alloc] call {i}: B={w.B} H={w.H} lengths={w.n_tokens}")
        M = len(w.ckpt_pos[0])
        outs = [(torch.full((w.B, M, w.H, 128, 128), float("nan"), device="cuda"),
                 torch.full((w.B, w.H, 128, 128), float("nan"), device="cuda"),
                 torch.full_like(w.v, float("nan"))) for _ in range(2)]
        ws = torch.empty(gdn.prefill_split_workspace_bytes(w.B, w.H, 128, 128), dtype=torch.uint8, device="cuda")
        torch.cuda.synchronize()
        free0 = torch.cuda.mem_get_info()[0]
        C0, S0, O0 = gdn.prefill_emit_checkpoints_split_noalloc(w.q, w.k, w.v, w.alpha, w.beta, w.tok_offset,
                                                                w.ckpt_pos, flags=w.flags, ckpt_states=outs[0][0],
                                                                state_out=outs[0][1], o=outs[0][2])
        torch.cuda.synchronize()
        free1 = torch.cuda.mem_get_info()[0]
        # nothing of the workspace's size was allocated (the scratch is part of the loaded library)
        assert free0 - free1 < ws.numel() // 2, (free0, free1)
        C1, S1, O1 = gdn.prefill_emit_checkpoints_split(w.q, w.k, w.v, w.alpha, w.beta, w.tok_offset, w.ckpt_pos,
                                                        flags=w.flags, ckpt_states=outs[1][0],
                                                        state_out=outs[1][1], o=outs[1][2], workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(S0, S1) and torch.equal(C0, C1) and torch.equal(O0, O1)
        PT.check_batched(w, {"no-alloc": (S0, O0, C0)}, emit=PT.emit_for(w), label=f"no-alloc-{i}", log=_log)


def test_noalloc_split_prefill_refuses_inputs_beyond_the_scratch(gdn):
    w = _prefill(303, 1, 129, [900], 2)
    with pytest.raises(gdn.GDNError) as e:
        gdn.prefill_emit_checkpoints_split_noalloc(w.q, w.k, w.v, w.alpha, w.beta, w.tok_offset, w.ckpt_pos,
                                                   flags=w.flags)
    assert e.value.status == 2
