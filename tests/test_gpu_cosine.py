"""GPU parity of the cosine-dissimilarity metric switch (kvc_score_centroid with
KVC_METRIC_COSINE: s_t = 1 - cos(k_t, mu), the cosine-to-centroid baseline of the
ManifoldKV abstract) against the CPU oracle, through the C ABI.  Rules as for the
L2 score: fp32 scores within rel 1e-4 (+1e-6 rms); retained sets identical except
for tokens within that tolerance of the k-th score; gathered rows bit-exact."""
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import oracle
import synth
from tests.helpers import index_sets_agree, score_close
from token_scoring_eviction_amd import kvc

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _check(K, s, W=None):
    bits = synth.bf16_bits(K)
    ora, mu = oracle.score_cosine(bits) if W is None else oracle.score_cosine_windowed(bits, W)
    ok, rel, nbad = score_close(s.cpu().numpy(), ora)
    assert ok, "cosine scores: %d outside tolerance, max rel %.3g" % (nbad, rel)
    return ora, mu


@pytest.mark.parametrize("path", ["0", "1"])
@pytest.mark.parametrize("G,S", [(1, 1), (3, 257), (2, 1000), (4, 4096), (1, 16384 + 77)])
def test_cosine_global_small(gpu_lib, kvc_option, G, S, path):
    kvc_option("score_path", 1 + int(path))
    K, _, _ = synth.manifold_global(1, 1, G, S, planted=min(4, S), seed=S + 1, device=DEV)
    mu_gpu = torch.empty((G, 128), dtype=torch.float32, device=DEV)
    s = gpu_lib.kvc_score_centroid(K, metric="cosine", centroids=mu_gpu)
    torch.cuda.synchronize()
    _, mu = _check(K, s)
    # the centroid output is the mean itself, not its direction
    np.testing.assert_allclose(mu_gpu.cpu().numpy(), mu, rtol=1e-5, atol=1e-5)


@pytest.mark.parametrize("path", ["0", "1"])
@pytest.mark.parametrize("S,W", [(1000, 1), (1000, 300), (4096 * 3 + 5, 4096), (8192, 512)])
def test_cosine_windowed_small(gpu_lib, kvc_option, S, W, path):
    kvc_option("score_path", 1 + int(path))
    K, _ = synth.manifold_drifting(1, 1, 2, S, segment=max(1, S // 3), seed=W + 7, device=DEV)
    s = gpu_lib.kvc_score_centroid(K, W=W, metric="cosine")
    torch.cuda.synchronize()
    _check(K, s, W)


def test_cosine_degenerate_and_nearly_parallel(gpu_lib, kvc_option):
    # slice 0: a zero key among keys with a nonzero centroid (score 1);
    # slice 1: integer keys summing exactly to zero (zero centroid: every score 1);
    # slice 2: keys nearly parallel to the centroid (scores ~1e-5, which the evaluation
    #          as a squared distance of unit vectors keeps to rel 1e-4)
    S = 600
    rng = np.random.default_rng(3)
    K = np.zeros((3, S, 128), np.float32)
    K[0] = rng.normal(1.0, 1.0, (S, 128))
    K[0, 17] = 0.0
    half = rng.integers(-20, 21, (S // 2, 128)).astype(np.float32)
    K[1, :S // 2], K[1, S // 2:] = half, -half
    base = rng.normal(0.0, 1.0, 128)
    K[2] = base[None] * rng.uniform(0.5, 2.0, (S, 1)) + rng.normal(0.0, 4e-3, (S, 128))
    Kt = torch.from_numpy(K).to(torch.bfloat16).to(DEV)
    for path in ("0", "1"):
        kvc_option("score_path", 1 + int(path))
        s = gpu_lib.kvc_score_centroid(Kt, metric="cosine")
        torch.cuda.synchronize()
        ora, _ = _check(Kt, s)
        sc = s.cpu().numpy()
        assert sc[0, 17] == 1.0 and np.all(sc[1] == 1.0)
        assert ora[2].max() < 1e-3  # the nearly parallel slice really is nearly parallel


@pytest.mark.parametrize("W", [None, 4096, 1000])
def test_cosine_fused_and_three_launch_paths_agree(gpu_lib, kvc_option, W):
    K, _, _ = synth.manifold_global(4, 1, 8, 12288 + 100, planted=8, seed=5, device=DEV)
    kvc_option("score_path", 1)
    f = gpu_lib.kvc_score_centroid(K, W=W, metric="cosine").clone()
    kvc_option("score_path", 2)
    u = gpu_lib.kvc_score_centroid(K, W=W, metric="cosine")
    torch.cuda.synchronize()
    for x in (f, u):
        _check(K, x, W)


def test_l2_metric_is_the_l2_entry_point(gpu_lib):
    K, _, _ = synth.manifold_global(2, 1, 8, 5000, planted=8, seed=9, device=DEV)
    a = gpu_lib.kvc_score_l2(K).clone()
    b = gpu_lib.kvc_score_centroid(K, metric="l2").clone()
    c = gpu_lib.kvc_score_l2_windowed(K, 1024).clone()
    d = gpu_lib.kvc_score_centroid(K, W=1024, metric="l2")
    torch.cuda.synchronize()
    assert torch.equal(a, b) and torch.equal(c, d)


def test_unknown_metric_rejected(gpu_lib):
    K = torch.zeros((1, 16, 128), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(kvc.KvcError):
        gpu_lib.kvc_score_centroid(K, metric=7)


def test_cosine_eviction_llama_shape_full(gpu_lib):
    # the global-eviction workload (32 layers x 8 kv heads, S=16384, keep 8192) with the
    # cosine metric; every slice checked: scores, retained set, gathered rows
    K, V, _ = synth.manifold_global(32, 1, 8, 16384, planted=64, device=DEV)
    s = gpu_lib.kvc_score_centroid(K, metric="cosine")
    idx, Ko, Vo = gpu_lib.kvc_topk_compact(s, 8192, K, V)
    torch.cuda.synchronize()
    kb, vb = synth.bf16_bits(K), synth.bf16_bits(V)
    s_all, idx_all = s.cpu().numpy(), idx.cpu().numpy()
    ko, vo = synth.bf16_bits(Ko), synth.bf16_bits(Vo)

    def check(g):
        ora, _ = oracle.score_cosine(kb[g:g + 1])
        ok, rel, nbad = score_close(s_all[g:g + 1], ora)
        assert ok, "slice %d: %d scores off (max rel %.3g)" % (g, nbad, rel)
        o32 = ora.astype(np.float32)
        ok, _ = index_sets_agree(idx_all[g:g + 1], oracle.topk(o32, 8192), o32, 8192)
        assert ok, "slice %d: retained set differs beyond the threshold band" % g
        sel = idx_all[g].astype(np.int64)
        np.testing.assert_array_equal(ko[g], kb[g][sel])
        np.testing.assert_array_equal(vo[g], vb[g][sel])

    with ThreadPoolExecutor(max_workers=8) as ex:
        list(ex.map(check, range(K.shape[0])))
