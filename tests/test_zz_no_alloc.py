"""The allocation-free scoring entry point (kvc_score_centroid_noalloc, for callers
that cannot allocate device memory) against the workspace entry point
kvc_score_centroid it shares its kernels with: bit-identical scores and centroids
on two calls in a row, the second with a smaller input (so stale scratch contents
from the first must not leak into it), on both scoring paths and both metrics;
shapes beyond its fixed scratch are refused before anything is launched."""
import ctypes

import pytest
import torch

import synth

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _both(gpu_lib, K, W, metric):
    G, S, _ = K.shape
    nwin = 1 if W is None else -(-S // W)
    mu_a = torch.full((G, nwin, 128), 7.0, device=DEV)
    mu_b = torch.full((G, nwin, 128), -7.0, device=DEV)
    a = gpu_lib.kvc_score_centroid(K, W=W, metric=metric, centroids=mu_a)
    b = gpu_lib.kvc_score_centroid_noalloc(K, W=W, metric=metric, centroids=mu_b)
    torch.cuda.synchronize()
    return a, b, mu_a, mu_b


@pytest.mark.parametrize("metric", ["l2", "cosine"])
def test_noalloc_matches_workspace_entry_point(gpu_lib, metric):
    # first call: 64 slices x 16384 tokens (256 MiB of keys: the single-read kernel);
    # second call: 8 slices x 3000 tokens with 700-token windows (the
    # three-launch path), after the first left its scratch filled
    K1, _, _ = synth.manifold_global(8, 1, 8, 16384, planted=16, seed=51, device=DEV)
    K2, _ = synth.manifold_drifting(1, 1, 8, 3000, segment=1000, seed=52, device=DEV)
    for K, W in ((K1, None), (K2, 700)):
        a, b, mu_a, mu_b = _both(gpu_lib, K, W, metric)
        assert not torch.isnan(a).any()
        assert torch.equal(a.view(torch.int32), b.view(torch.int32))
        assert torch.equal(mu_a.view(torch.int32), mu_b.view(torch.int32))


def test_noalloc_both_paths_and_repeat(gpu_lib, kvc_option):
    K, _, _ = synth.manifold_global(2, 1, 8, 12288 + 100, planted=8, seed=53, device=DEV)
    small = K[:3, :2000].contiguous()
    for path in (1, 2):
        kvc_option("score_path", path)
        for X, W in ((K, 4096), (small, None), (K, None)):
            a, b, mu_a, mu_b = _both(gpu_lib, X, W, "l2")
            assert torch.equal(a.view(torch.int32), b.view(torch.int32)), (path, X.shape, W)
            assert torch.equal(mu_a.view(torch.int32), mu_b.view(torch.int32))


def test_noalloc_refuses_shapes_beyond_its_scratch(gpu_lib):
    lib = gpu_lib.load()
    K = torch.zeros((1, 256, 128), dtype=torch.bfloat16, device=DEV)
    s = torch.zeros((1, 256), dtype=torch.float32, device=DEV)
    p = lambda t: ctypes.c_void_p(t.data_ptr())
    # 1024 slices x 65536 tokens in 256-token windows would need ~384 MiB of scratch;
    # refused before any launch (the pointers are never read)
    st = lib.kvc_score_centroid_noalloc(p(K), 1024, 65536, 128, 256, 0, p(s), None, None)
    assert st == gpu_lib.ERR_WORKSPACE_TOO_SMALL
    assert lib.kvc_score_centroid_noalloc(p(K), 1, 256, 128, 0, 0, p(s), None, None) == gpu_lib.ERR_INVALID_ARGUMENT
    assert lib.kvc_score_centroid_noalloc(p(K), 1, 256, 128, 256, 5, p(s), None, None) == gpu_lib.ERR_INVALID_ARGUMENT
    torch.cuda.synchronize()
