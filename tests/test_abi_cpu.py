"""Host-side checks of the C ABI (no GPU, no compute call): the library loads,
exports every function include/kvc.h declares, reports its version and status
texts, and sizes workspaces consistently."""
import ctypes
import os
import re

import pytest

from tests.helpers import built_library
from token_scoring_eviction_amd import kvc

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "kvc.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kvc_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_abi():
    assert _declared() == sorted(kvc.EXPORTED)


def test_library_exports_every_declared_symbol():
    if not built_library():
        pytest.skip("hipcc is not installed here")
    lib = kvc.load()
    for name in _declared():
        assert hasattr(lib, name), name
    assert lib.kvc_abi_version() == 5
    assert lib.kvc_status_str(kvc.OK) == b"ok"
    assert lib.kvc_status_str(kvc.ERR_WORKSPACE_TOO_SMALL) == b"workspace too small"
    assert lib.kvc_status_str(99) == b"unknown status"


def test_workspace_sizing():
    if not built_library():
        pytest.skip("hipcc is not installed here")
    D = kvc.Dims
    # global and windowed scoring: per-chunk partials plus per-window centroids
    g1 = kvc.workspace_bytes(kvc.OP_SCORE_L2, D(1, 1, 256, 0, 16384, 0, 128, 0, 0))
    assert g1 >= 256 * (16384 // 256) * 128 * 4
    w = [kvc.workspace_bytes(kvc.OP_SCORE_L2_WINDOWED, D(1, 1, 256, 0, 65536, 0, 128, 0, 0), 0, W)
         for W in (1024, 4096, 65536)]
    assert all(x > 0 for x in w)
    # monotone in the number of slices
    a = kvc.workspace_bytes(kvc.OP_SCORE_L2, D(1, 1, 8, 0, 4096, 0, 128, 0, 0))
    b = kvc.workspace_bytes(kvc.OP_SCORE_L2, D(1, 1, 16, 0, 4096, 0, 128, 0, 0))
    assert 0 < a < b
    # compress needs folded query fragments only when a window is given (two bf16 terms
    # per element for a 128-query window, three below 32 queries)
    assert kvc.workspace_bytes(kvc.OP_LOWRANK_COMPRESS, D(32, 4, 8, 32, 32768, 0, 128, 64, 32)) == \
        1024 * 4 * 8 * 2 * 64 * 16
    assert kvc.workspace_bytes(kvc.OP_LOWRANK_COMPRESS, D(1, 1, 2, 2, 100, 0, 128, 64, 1)) == \
        2 * 1 * 8 * 3 * 64 * 16
    assert kvc.workspace_bytes(kvc.OP_LOWRANK_COMPRESS, D(32, 4, 8, 0, 32768, 0, 128, 64, 0)) == 0
    # invalid or unsupported shapes report 0
    assert kvc.workspace_bytes(kvc.OP_LOWRANK_COMPRESS, D(1, 1, 1, 0, 10, 0, 64, 32, 0)) == 0
    assert kvc.workspace_bytes(kvc.OP_OJA_UPDATE, D(1, 1, 1, 0, 10, 0, 128, 48, 0), 0, 1) == 0
    assert kvc.workspace_bytes(kvc.OP_OJA_UPDATE, D(32, 1, 8, 0, 131072, 0, 128, 64, 0), 0, 32) > 0
    assert kvc.workspace_bytes(kvc.OP_TOPK_COMPACT, D(1, 1, 8, 0, 4096, 0, 128, 0, 0), 3277) == 0
    # ragged selection: the status header, then a budget and an offset per slice
    assert kvc.workspace_bytes(kvc.OP_TOPK_RAGGED, D(1, 1, 300, 0, 4096, 0, 128, 0, 0)) == \
        256 + 2560 + 300 * 8  # 2400 bytes of budgets padded to 2560, then the offsets
    assert kvc.workspace_bytes(kvc.OP_RECONSTRUCT, D(1, 1, 8, 0, 4096, 0, 128, 64, 0), 10) == 0
    assert kvc.load().kvc_workspace_bytes(0, None, 0, 0) == 0
