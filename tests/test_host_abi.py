"""CPU checks of the C ABI: the library loads, exports every function the
header declares, and its host-only logic (exact span selection, argument
validation) behaves as documented.  No kernel is launched here: every call
below returns before any HIP API is touched."""
import ctypes
import json
import os
import re

import numpy as np
import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gdnreplay.h")


@pytest.fixture(scope="module")
def gdn():
    import gated_delta_rule_scan_amd as g
    if not os.path.exists(g.library_path()):
        from gated_delta_rule_scan_amd.build import build
        build()
    return g


def _declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(gdn_[a-z_]+)\s*\(", src)))


def test_exports_every_declared_function(gdn):
    names = _declared_functions()
    assert {"gdn_tail_replay", "gdn_resume", "gdn_prefill_emit_checkpoints"} <= set(names)
    lib = ctypes.CDLL(gdn.library_path())
    for n in names:
        assert hasattr(lib, n), n


def test_header_compiles_as_c():
    """The header is plain C: it compiles with gcc without HIP headers."""
    import subprocess
    import tempfile
    with tempfile.TemporaryDirectory() as d:
        c = os.path.join(d, "t.c")
        open(c, "w").write('#include "gdnreplay.h"\nint main(void){gdn_shape s={0};(void)s;return 0;}\n')
        subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-I", os.path.join(ROOT, "include"),
                        "-c", c, "-o", os.path.join(d, "t.o")], check=True)


def test_version(gdn):
    assert gdn.version().startswith("libgdnreplay")


def test_tail_len_golden_and_exact(gdn):
    g = json.load(open(os.path.join(ROOT, "tests", "golden", "tail_worked_example.json")))
    assert gdn.tail_len(g["m"], g["r_num"], g["r_den"]) == g["k"]
    assert gdn.tail_len(32768, 5, 100) == 1639
    assert gdn.tail_len(32768, 10, 100) == 3277
    for m in list(range(0, 300)) + [65535, 65536, 2 ** 40]:
        for num, den in [(5, 100), (10, 100), (1, 3), (2, 7), (0, 1), (3, 2)]:
            assert gdn.tail_len(m, num, den) == oracle.tail_length(m, num, den)
    # m * r_num beyond 64 bits is still exact
    assert gdn.tail_len(2 ** 62, 3, 4) == 3 * 2 ** 60
    assert gdn.tail_len(-1, 1, 2) == -1
    assert gdn.tail_len(5, -1, 2) == -1
    assert gdn.tail_len(5, 1, 0) == -1


def test_select_checkpoint_brute_force(gdn):
    rng = np.random.default_rng(0)
    for _ in range(100):
        N = int(rng.integers(1, 60))
        M = int(rng.integers(0, min(N, 9) + 1))
        pos = sorted(int(x) + 1 for x in rng.choice(N, M, replace=False))
        for d in range(0, N + 1):
            assert gdn.select_checkpoint(pos, d) == oracle.select_checkpoint(pos, d)
    assert gdn.select_checkpoint([3, 3], 5) == -1
    assert gdn.select_checkpoint([0, 3], 5) == -1
    assert gdn.select_checkpoint([1, 3], -1) == -1


def test_kernel_selection(gdn):
    import torch
    assert gdn.kernel_for(1, 1, 16, 16, torch.float32) == "recurrent"
    assert gdn.kernel_for(1, 1, 128, 128, torch.bfloat16, gdn.KERNEL_RECURRENT) == "recurrent"
    with pytest.raises(gdn.GDNError):
        gdn.kernel_for(1, 1, 128, 128, torch.float32, gdn.KERNEL_CHUNKED)
    with pytest.raises(gdn.GDNError):
        gdn.kernel_for(1, 1, 96, 128, torch.bfloat16)
