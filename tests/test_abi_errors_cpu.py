"""Host-side argument checks of the C ABI (no GPU needed): every entry point
validates its arguments synchronously and returns a status before any HIP call,
so bad shapes, missing buffers, misaligned pointers and short workspaces are
rejected here with the documented codes, and empty work returns KVC_OK.  The
device pointers below are placeholder addresses that are never dereferenced."""
import ctypes
import math
import os

import numpy as np
import pytest

from tests.helpers import built_library
from token_scoring_eviction_amd import kvc

pytestmark = pytest.mark.skipif(not built_library(), reason="hipcc is not installed here")

OK, INV, UNS, WS = kvc.OK, kvc.ERR_INVALID_ARGUMENT, kvc.ERR_UNSUPPORTED, kvc.ERR_WORKSPACE_TOO_SMALL
NULL = None


def P(addr):
    """A placeholder device address (16-byte aligned unless chosen otherwise)."""
    return ctypes.c_void_p(addr)


A, B, C, D_, E, F, W_ = (P(0x100000 * i) for i in range(1, 8))


def dims(L=1, B=1, H_kv=2, H_q=8, S=100, S_stride=0, D=128, R=64, W_q=4):
    return ctypes.byref(kvc.Dims(L, B, H_kv, H_q, S, S_stride, D, R, W_q))


@pytest.fixture(scope="module")
def lib():
    return kvc.load()


def test_score_entry_points(lib):
    f = lib.kvc_score_l2
    assert f(A, -1, 100, 128, B, NULL, W_, 1 << 20, NULL) == INV
    assert f(A, 2, 0, 128, B, NULL, W_, 1 << 20, NULL) == INV
    assert f(A, 2, 100, 64, B, NULL, W_, 1 << 20, NULL) == UNS
    assert f(A, 0, 100, 128, B, NULL, W_, 0, NULL) == OK          # no slices: nothing to do
    assert f(NULL, 2, 100, 128, B, NULL, W_, 1 << 20, NULL) == INV
    assert f(P(0x100002), 2, 100, 128, B, NULL, W_, 1 << 20, NULL) == INV  # K not 16-byte aligned
    assert f(A, 2, 100, 128, B, NULL, W_, 0, NULL) == WS
    assert lib.kvc_score_l2_windowed(A, 2, 100, 128, 0, B, NULL, W_, 1 << 20, NULL) == INV
    assert lib.kvc_score_centroid(A, 2, 100, 128, 100, 7, B, NULL, W_, 1 << 20, NULL) == INV  # metric


def test_topk_entry_points(lib):
    f = lib.kvc_topk_compact
    assert f(A, 2, 100, 100, 101, NULL, NULL, 128, B, NULL, NULL, NULL, 0, NULL) == INV  # k > S
    assert f(A, 2, 100, 99, 10, NULL, NULL, 128, B, NULL, NULL, NULL, 0, NULL) == INV   # stride < S
    assert f(A, 2, 100, 100, 10, C, NULL, 128, B, NULL, NULL, NULL, 0, NULL) == INV     # K without K_out
    assert f(A, 2, 100, 100, 10, C, NULL, 64, B, D_, NULL, NULL, 0, NULL) == UNS        # D != 128
    assert f(A, 2, 100, 100, 0, NULL, NULL, 128, B, NULL, NULL, NULL, 0, NULL) == OK    # k = 0
    assert f(A, 2, 100, 100, 0, C, C, 128, B, NULL, NULL, NULL, 0, NULL) == OK          # k = 0: no row outputs needed
    assert f(A, 0, 100, 100, 10, NULL, NULL, 128, B, NULL, NULL, NULL, 0, NULL) == OK   # G = 0
    assert f(NULL, 2, 100, 100, 10, NULL, NULL, 128, B, NULL, NULL, NULL, 0, NULL) == INV
    assert f(A, 2, 100, 100, 10, P(0x100008), NULL, 128, B, D_, NULL, NULL, 0, NULL) == INV  # K misaligned
    # budgets are a device array checked by the call's kernels; the host checks their bound
    # k_max, the packed capacity k_total, the pointers and the workspace
    g = lib.kvc_topk_compact_ragged
    assert g(A, 2, 100, 100, C, 101, 10, NULL, NULL, 128, B, NULL, NULL, W_, 1 << 20, NULL) == INV  # k_max > S
    assert g(A, 2, 100, 100, C, 5, -1, NULL, NULL, 128, B, NULL, NULL, W_, 1 << 20, NULL) == INV    # k_total < 0
    assert g(A, 2, 100, 100, NULL, 5, 10, NULL, NULL, 128, B, NULL, NULL, W_, 1 << 20, NULL) == INV  # no budgets
    assert g(A, 2, 100, 100, P(0x300004), 5, 10, NULL, NULL, 128, B, NULL, NULL, W_, 1 << 20,
             NULL) == INV                                                                     # budgets misaligned
    assert g(A, 2, 100, 100, C, 5, 10, NULL, NULL, 128, B, NULL, NULL, NULL, 0, NULL) == INV    # no workspace
    assert g(A, 2, 100, 100, C, 5, 10, NULL, NULL, 128, B, NULL, NULL, W_, 0, NULL) == WS
    assert g(A, 0, 100, 100, C, 5, 10, NULL, NULL, 128, B, NULL, NULL, NULL, 0, NULL) == OK     # G = 0


def test_lowrank_entry_points(lib):
    f = lib.kvc_lowrank_compress
    args = (A, B, C, D_, E, F, P(0x800000), P(0x900000), W_, 1 << 24, NULL)
    assert f(None, *args) == INV
    assert f(dims(D=64, R=32), *args) == UNS
    assert f(dims(R=48), *args) == UNS
    assert f(dims(R=256), *args) == INV                           # R > D
    assert f(dims(H_q=6, H_kv=4), *args) == INV                   # H_q not a multiple of H_kv
    assert f(dims(), A, B, C, D_, E, F, P(0x800000), NULL, W_, 1 << 24, NULL) == INV  # window, no err
    assert f(dims(), A, B, NULL, D_, E, F, NULL, NULL, W_, 1 << 24, NULL) == INV      # V, no V~
    assert f(dims(), A, B, C, D_, E, F, P(0x800000), P(0x900000), W_, 0, NULL) == WS
    assert f(dims(S=0), *args) == OK                              # no tokens
    g = lib.kvc_lowrank_compress_reconstruct
    assert g(dims(), A, B, C, D_, E, F, P(0x800000), P(0x900000), NULL, P(0xa00000), W_, 1 << 24,
             NULL) == INV                                         # K^ missing
    assert g(dims(), A, B, C, D_, E, F, P(0x800000), P(0x900000), P(0xb00000), NULL, W_, 1 << 24,
             NULL) == INV                                         # V given, V^ missing
    h = lib.kvc_reconstruct
    assert h(dims(S=100), A, B, NULL, NULL, 101, C, NULL, 0, NULL) == INV  # k > S
    assert h(dims(S=100), A, B, NULL, NULL, 5, C, NULL, 0, NULL) == INV    # anchors missing
    p = lib.kvc_place_anchors
    assert p(dims(S=100), A, B, 101, C, NULL) == INV
    assert p(dims(S=100, D=64, R=32), A, B, 5, C, NULL) == UNS
    assert p(dims(S=100), NULL, NULL, 0, NULL, NULL) == OK        # no anchors
    assert lib.kvc_place_anchors_bf16(dims(S=100), A, NULL, 5, C, NULL) == INV


def test_oja_and_append_entry_points(lib):
    f = lib.kvc_oja_update
    assert f(dims(), A, B, 0, 1e-3, W_, 1 << 24, NULL) == INV      # pool < 1
    assert f(dims(), A, B, 32, math.nan, W_, 1 << 24, NULL) == INV
    assert f(dims(R=48), A, B, 32, 1e-3, W_, 1 << 24, NULL) == UNS
    assert f(dims(B=0), A, B, 32, 1e-3, W_, 1 << 24, NULL) == INV
    assert f(dims(), A, B, 32, 1e-3, W_, 0, NULL) == WS
    g = lib.kvc_decode_append
    row = (A, B, NULL, C, D_, NULL, NULL, NULL)
    assert g(dims(S=100), 100, 32, 0, *row, NULL) == INV           # pos past the cache
    assert g(dims(S=100), 10, 32, 32, *row, NULL) == INV           # slot past the buffer
    assert g(dims(S=100, D=64), 10, 32, 0, *row, NULL) == UNS
    assert g(dims(S=100), 10, 32, 0, A, B, NULL, C, D_, E, NULL, NULL, NULL) == INV  # K_buf without V_buf


def test_refine_entry_points(lib):
    f = lib.kvc_cluster_summaries
    assert f(A, B, 2, 100, 128, 0, C, D_, E, F, NULL) == INV       # c = 0
    assert f(A, B, 2, 100, 64, 10, C, D_, E, F, NULL) == UNS
    assert f(A, B, 0, 100, 128, 10, C, D_, E, F, NULL) == OK
    assert f(NULL, B, 2, 100, 128, 10, C, D_, E, F, NULL) == INV
    g = lib.kvc_refine_risk
    assert g(A, B, C, 2, 100, 10, 128, D_, 9, E, W_, 1 << 20, NULL) == UNS   # more than 8 queries
    assert g(A, B, C, 2, 100, 10, 128, D_, 0, E, W_, 1 << 20, NULL) == OK    # no queries
    assert g(A, B, C, 2, 100, 10, 128, D_, -1, E, W_, 1 << 20, NULL) == INV
    assert g(A, B, C, 2, 100, 10, 128, D_, 4, E, NULL, 1 << 20, NULL) == INV  # no workspace
    assert g(A, B, C, 2, 100, 10, 128, P(0x400008), 4, E, W_, 1 << 20, NULL) == INV  # Q not 16-byte aligned
    need = kvc.workspace_bytes(kvc.OP_REFINE_RISK, kvc._dims(1, 1, 2, 0, 100, 0, 128, 0, 0), 10)
    assert need == 2 * 9 * 16                                     # one chunk record per slice
    assert g(A, B, C, 2, 100, 10, 128, D_, 4, E, W_, need - 1, NULL) == WS


def test_options_and_deferred_status(lib):
    # every option takes its documented range and nothing else (values unchanged on error)
    for opt, good, bad in ((kvc.OPTION_SCORE_PATH, (0, 1, 2), (-1, 3)),
                           (kvc.OPTION_SCORE_SPIN_LIMIT, (-1, 0, 2 ** 32 - 1), (-2, 2 ** 32)),
                           (kvc.OPTION_GATHER_PATH, (0, 1), (-1, 2))):
        for v in good:
            assert lib.kvc_set_option(opt, v) == OK
        for v in bad:
            assert lib.kvc_set_option(opt, v) == INV
    assert lib.kvc_set_option(7, 0) == INV
    for name, v in kvc.OPTION_DEFAULTS.items():
        assert lib.kvc_set_option(kvc.OPTIONS[name], v) == OK
    # the status query refuses a missing or misaligned workspace before touching the device
    assert lib.kvc_workspace_status(NULL, NULL) == INV
    assert lib.kvc_workspace_status(P(0x100010), NULL) == INV
    assert lib.kvc_status_str(kvc.ERR_WAIT_EXPIRED).startswith(b"an in-kernel wait expired")
