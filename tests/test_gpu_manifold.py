"""GPU parity of ManifoldKV scoring (global and windowed), retention and
compaction against the CPU oracle, through the C ABI.  Rules: fp32 scores
within rel 1e-4 (+1e-6 rms); top-k on identical fp32 scores bit-exact;
end-to-end retained sets identical except for tokens within rel 1e-4 of the
k-th score; gathered rows bit-exact."""
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import oracle
import synth
from tests.helpers import index_sets_agree, score_close

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _scores_vs_oracle(K, gpu_scores, W=None):
    bits = synth.bf16_bits(K)
    ora, mu = oracle.score_l2(bits) if W is None else oracle.score_l2_windowed(bits, W)
    ok, rel, nbad = score_close(gpu_scores.cpu().numpy(), ora)
    assert ok, "scores: %d outside tolerance, max rel %.3g" % (nbad, rel)
    return ora, mu


# path "0": the single-read kernel, "1": the three-launch path (caches under 12 MiB
# take the latter by default); chosen with the score_path option.  Slices of more
# than 32 tiles (8192 tokens) split the centroid gather over 2, 4, ... aggregators:
# 16461 tokens are 65 tiles (4 aggregators), 40000 are 157 (8), 131149 are 513 (16,
# with 8 tiles per poll above 256 tiles)
@pytest.mark.parametrize("path", ["0", "1"])
@pytest.mark.parametrize("G,S", [(1, 1), (3, 257), (2, 1000), (4, 4096), (1, 16384 + 77), (2, 40000),
                                 (1, 131072 + 77)])
def test_score_l2_small(gpu_lib, kvc_option, G, S, path):
    kvc_option("score_path", 1 + int(path))
    K, _, _ = synth.manifold_global(1, 1, G, S, planted=min(4, S), seed=S, device=DEV)
    mu_gpu = torch.empty((G, 128), dtype=torch.float32, device=DEV)
    s = gpu_lib.kvc_score_l2(K, centroid=mu_gpu)
    torch.cuda.synchronize()
    _, mu = _scores_vs_oracle(K, s)
    np.testing.assert_allclose(mu_gpu.cpu().numpy(), mu, rtol=1e-5, atol=1e-5)


# windows of 32 tiles or more (8192 tokens and up) take the single-read kernel's early-publish
# order; the last window of a slice may be short
@pytest.mark.parametrize("S,W", [(1000, 1), (1000, 1000), (1000, 5000), (1000, 300), (4096 * 3 + 5, 4096),
                                 (8192, 512), (20000, 8192), (30000, 9000)])
@pytest.mark.parametrize("path", ["0", "1"])
def test_score_l2_windowed_small(gpu_lib, kvc_option, S, W, path):
    kvc_option("score_path", 1 + int(path))
    K, _ = synth.manifold_drifting(1, 1, 2, S, segment=max(1, S // 3), seed=W, device=DEV)
    nwin = -(-S // W)
    mu_gpu = torch.empty((2, nwin, 128), dtype=torch.float32, device=DEV)
    s = gpu_lib.kvc_score_l2_windowed(K, W, centroids=mu_gpu)
    torch.cuda.synchronize()
    _, mu = _scores_vs_oracle(K, s, W)
    np.testing.assert_allclose(mu_gpu.cpu().numpy(), mu, rtol=1e-5, atol=1e-5)
    if W == 1:
        assert torch.all(s == 0)


@pytest.mark.parametrize("kind", ["normal", "ties", "signed"])
# slice lengths for every register-held select instance (up to 1, 2, 4, 8 and 16 tiles of
# 4096 keys) and both sides of the longest one (65536 held; 65537 and the decode loop's
# 131104 hold the first 49152 and read the rest at every pass)
@pytest.mark.parametrize("G,S", [(1, 1), (3, 100), (2, 4096), (2, 4097), (2, 16384), (5, 20000),
                                 (1, 65536), (1, 65537), (2, 131104)])
def test_topk_bit_exact_on_same_scores(gpu_lib, kind, G, S):
    s = synth.random_scores(G, S, seed=S * 7 + G, kind=kind, device="cpu")
    s_gpu = s.to(DEV)
    for k in sorted({0, 1, S // 3, S // 2, S - 1, S}):
        if k < 0:
            continue
        idx, _, _ = gpu_lib.kvc_topk_compact(s_gpu, k)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(idx.cpu().numpy(), oracle.topk(s.numpy(), k))


def test_topk_strided_and_gather_bit_exact(gpu_lib):
    G, S, stride, k = 3, 5000, 5123, 1234
    K = torch.randint(-32768, 32767, (G, stride, 128), dtype=torch.int16, device=DEV).view(torch.bfloat16)
    V = torch.randint(-32768, 32767, (G, stride, 128), dtype=torch.int16, device=DEV).view(torch.bfloat16)
    s = synth.random_scores(G, stride, seed=5, device="cpu")
    idx, Ko, Vo = gpu_lib.kvc_topk_compact(s.to(DEV), k, K, V, S=S)
    torch.cuda.synchronize()
    ref_idx = oracle.topk(s.numpy(), k, S=S)
    np.testing.assert_array_equal(idx.cpu().numpy(), ref_idx)
    np.testing.assert_array_equal(synth.bf16_bits(Ko), oracle.gather(synth.bf16_bits(K), ref_idx, S=S))
    np.testing.assert_array_equal(synth.bf16_bits(Vo), oracle.gather(synth.bf16_bits(V), ref_idx, S=S))


@pytest.mark.parametrize("separate", [False, True])
def test_gather_paths_bit_exact(gpu_lib, kvc_option, separate):
    # 300 slices (more than one per compute unit, so gather_path 1 has the selecting
    # workgroup copy the rows itself; 0 selects the wide gather, the default), ragged S,
    # strided cache, k from 1 to S including the 8192-row boundary of the in-workgroup copy
    G, S, stride = 300, 8197, 8200
    kvc_option("gather_path", 0 if separate else 1)
    K = torch.randint(-32768, 32767, (G, stride, 128), dtype=torch.int16, device=DEV).view(torch.bfloat16)
    V = torch.randint(-32768, 32767, (G, stride, 128), dtype=torch.int16, device=DEV).view(torch.bfloat16)
    s = synth.random_scores(G, stride, seed=11, kind="ties", device="cpu")
    Kb, Vb = synth.bf16_bits(K), synth.bf16_bits(V)
    for k in (1, 777, 8192, 8193, S):
        idx, Ko, Vo = gpu_lib.kvc_topk_compact(s.to(DEV), k, K, V, S=S)
        torch.cuda.synchronize()
        ref_idx = oracle.topk(s.numpy(), k, S=S)
        np.testing.assert_array_equal(idx.cpu().numpy(), ref_idx)
        np.testing.assert_array_equal(synth.bf16_bits(Ko), oracle.gather(Kb, ref_idx, S=S))
        np.testing.assert_array_equal(synth.bf16_bits(Vo), oracle.gather(Vb, ref_idx, S=S))


def _evict_and_check(gpu_lib, K, V, keep, W=None, slices=None, threads=8):
    s = gpu_lib.kvc_score_l2(K) if W is None else gpu_lib.kvc_score_l2_windowed(K, W)
    idx, Ko, Vo = gpu_lib.kvc_topk_compact(s, keep, K, V)
    torch.cuda.synchronize()
    slices = list(range(K.shape[0]) if slices is None else slices)
    kb_all, vb_all = synth.bf16_bits(K), synth.bf16_bits(V)
    s_all, idx_all = s.cpu().numpy(), idx.cpu().numpy()
    ko_all, vo_all = synth.bf16_bits(Ko), synth.bf16_bits(Vo)

    def check(g):
        kb = kb_all[g:g + 1]
        ora, _ = oracle.score_l2(kb) if W is None else oracle.score_l2_windowed(kb, W)
        ok, rel, nbad = score_close(s_all[g:g + 1], ora)
        assert ok, "slice %d: %d scores off (max rel %.3g)" % (g, nbad, rel)
        ora32 = ora.astype(np.float32)
        ora_idx = oracle.topk(ora32, keep)
        gi = idx_all[g:g + 1]
        ok, nb = index_sets_agree(gi, ora_idx, ora32, keep)
        assert ok, "slice %d: retained set differs beyond the threshold band" % g
        # gathered rows are the input rows at the GPU's indices, bit for bit
        # (a plain index_select on the host; the oracle never takes GPU output)
        sel = gi[0].astype(np.int64)
        np.testing.assert_array_equal(ko_all[g], kb[0][sel])
        np.testing.assert_array_equal(vo_all[g], vb_all[g][sel])
        return nb

    # the oracle is single-threaded C called through ctypes (the GIL is released),
    # so independent slices are checked concurrently
    with ThreadPoolExecutor(max_workers=threads) as ex:
        nb_total = sum(ex.map(check, slices))
    return idx, nb_total


def test_global_8x4096_keep3277_full(gpu_lib):
    # 1 layer x 8 kv heads, S=4096, drop 20% -> keep 3277; every slice checked
    K, V, plant = synth.manifold_global(1, 1, 8, 4096, planted=16, device=DEV)
    idx, _ = _evict_and_check(gpu_lib, K, V, oracle.keep_count(4096, 20))
    for g in range(8):  # the planted x4 tokens survive
        assert set(plant[g].tolist()) <= set(idx[g].cpu().tolist())


def test_global_256x16384_keep8192(gpu_lib):
    # 32 layers x 8 kv heads, S=16384, keep 8192, in the launch configuration the
    # benchmark times; every one of the 256 slices checked against the oracle
    K, V, plant = synth.manifold_global(32, 1, 8, 16384, planted=64, device=DEV)
    idx, _ = _evict_and_check(gpu_lib, K, V, 8192)
    for g in (0, 101, 255):  # the planted x4 tokens survive
        assert set(plant[g].tolist()) <= set(idx[g].cpu().tolist())


def test_windowed_256x65536_w4096_keep49152(gpu_lib):
    # 32 layers x 8 kv heads, S=65536, W=4096, keep 49152; every slice checked
    K, V = synth.manifold_drifting(32, 1, 8, 65536, device=DEV)
    _evict_and_check(gpu_lib, K, V, 49152, W=4096)


def test_determinism(gpu_lib):
    K, V, _ = synth.manifold_global(2, 1, 8, 8192, planted=8, device=DEV)
    a = gpu_lib.kvc_score_l2(K).clone()
    ia, Ka, _ = gpu_lib.kvc_topk_compact(a, 3000, K, V)
    b = gpu_lib.kvc_score_l2(K)
    ib, Kb, _ = gpu_lib.kvc_topk_compact(b, 3000, K, V)
    torch.cuda.synchronize()
    assert torch.equal(a, b) and torch.equal(ia, ib) and torch.equal(Ka.view(torch.int16), Kb.view(torch.int16))


@pytest.mark.parametrize("W", [None, 8500, 4096, 1000])
def test_fused_and_three_launch_paths_agree(gpu_lib, kvc_option, W):
    # the single-read path and the three-launch path compute the same scores
    K, _, _ = synth.manifold_global(4, 1, 8, 12288 + 100, planted=8, seed=3, device=DEV)
    kvc_option("score_path", 1)
    f = gpu_lib.kvc_score_l2(K) if W is None else gpu_lib.kvc_score_l2_windowed(K, W)
    f = f.clone()
    kvc_option("score_path", 2)
    u = gpu_lib.kvc_score_l2(K) if W is None else gpu_lib.kvc_score_l2_windowed(K, W)
    torch.cuda.synchronize()
    ora, _ = oracle.score_l2(synth.bf16_bits(K)) if W is None else oracle.score_l2_windowed(synth.bf16_bits(K), W)
    for x in (f, u):
        ok, rel, nbad = score_close(x.cpu().numpy(), ora)
        assert ok, (rel, nbad)


def test_binding_refuses_strided_and_host_tensors(gpu_lib):
    # the C ABI reads dense rows: a strided view or a host tensor is refused, not misread
    K = torch.zeros((4, 256, 128), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(ValueError):
        gpu_lib.kvc_score_l2(K[:, ::2])
    s = torch.rand((4, 256), device=DEV)
    with pytest.raises(ValueError):
        gpu_lib.kvc_topk_compact(s.t().contiguous().t(), 10)
    with pytest.raises(ValueError):
        gpu_lib.kvc_topk_compact(s, 10, K.cpu(), K.cpu())


def test_binding_workspace_per_stream(gpu_lib):
    # the binding's cached workspace is one buffer per (device, stream): calls on two
    # streams may overlap without sharing scratch; results match the default stream's
    from token_scoring_eviction_amd import kvc
    K, _, _ = synth.manifold_global(2, 1, 8, 4096, planted=8, seed=9, device=DEV)
    ref = gpu_lib.kvc_score_l2(K).clone()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    s1.wait_stream(torch.cuda.current_stream())
    s2.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s1):
        w1 = kvc.workspace(1024)
        a = gpu_lib.kvc_score_l2(K)
    with torch.cuda.stream(s2):
        w2 = kvc.workspace(1024)
        b = gpu_lib.kvc_score_l2(K)
    torch.cuda.synchronize()
    assert w1.data_ptr() != w2.data_ptr()
    assert torch.equal(a, ref) and torch.equal(b, ref)


@pytest.mark.parametrize("W", [None, 9000, 1000])
@pytest.mark.parametrize("metric", ["l2", "cosine"])
def test_expired_centroid_waits_are_repaired_bit_exactly(gpu_lib, kvc_option, metric, W):
    # the single-read kernel's centroid waits are bounded; a spin limit of 0 set from the
    # host makes nearly every wait give up at its first poll.  Those teams are flagged,
    # and the repair launch queued after the kernel recomputes their centroids and
    # scores from the keys: every score and centroid must come out bit-identical to a
    # run whose waits succeed, and the workspace status must report nothing
    K, _, _ = synth.manifold_global(4, 1, 8, 16384, planted=8, seed=5, device=DEV)
    kvc_option("score_path", 1)
    G, S = K.shape[0], K.shape[1]
    nwin = 1 if W is None else -(-S // W)

    def score():
        mu = torch.empty((G, nwin, 128), dtype=torch.float32, device=DEV)
        sc = gpu_lib.kvc_score_centroid(K, W=W, metric=metric, centroids=mu)
        return sc.clone(), mu

    ref, ref_mu = score()
    gpu_lib.kvc_workspace_status()
    kvc_option("score_spin_limit", 0)
    rep, rep_mu = score()
    gpu_lib.kvc_workspace_status()  # a repaired call reports no failure
    kvc_option("score_spin_limit", -1)
    again, _ = score()
    torch.cuda.synchronize()
    assert not torch.isnan(ref).any()
    assert torch.equal(rep, ref) and torch.equal(rep_mu, ref_mu)
    assert torch.equal(again, ref)


@pytest.mark.parametrize("G,S,W,metric", [(4, 40000, None, "l2"), (4, 40000, None, "cosine"),
                                          (2, 131072 + 300, None, "l2"), (3, 118016, None, "l2"),
                                          (4, 70000, 33000, "l2")])
def test_multi_aggregator_teams_repair_bit_exactly(gpu_lib, kvc_option, G, S, W, metric):
    # teams of more than 32 tiles gather their centroid with several aggregators, each
    # owning a block of channels (8 for the 157-tile slices of 40000 tokens and the
    # 129-tile windows of 33000; above 256 tiles one per 64 tiles: 8 for the 461-tile
    # slices of 118016, 16 for the 514-tile slices of 131372, whose member groups are
    # 5 tiles long).  The scores match
    # the oracle, and a run whose waits all give up is repaired to the same bits: the
    # repair launch adds the tile sums in the member groups the aggregators use
    K, _, _ = synth.manifold_global(1, 1, G, S, planted=8, seed=S % 1000, device=DEV)
    kvc_option("score_path", 1)
    nwin = 1 if W is None else -(-S // W)

    def score():
        mu = torch.empty((G, nwin, 128), dtype=torch.float32, device=DEV)
        sc = gpu_lib.kvc_score_centroid(K, W=W, metric=metric, centroids=mu)
        return sc.clone(), mu

    ref, ref_mu = score()
    torch.cuda.synchronize()
    if metric == "l2":
        _scores_vs_oracle(K, ref, W)
    kvc_option("score_spin_limit", 0)
    rep, rep_mu = score()
    gpu_lib.kvc_workspace_status()
    kvc_option("score_spin_limit", -1)
    torch.cuda.synchronize()
    assert not torch.isnan(ref).any()
    assert torch.equal(rep, ref) and torch.equal(rep_mu, ref_mu)


def test_scoring_beside_another_kernel_is_bit_identical(gpu_lib, kvc_option):
    # the single-read kernel is an ordinary launch: while a GEMM on a second stream holds
    # part of the GPU, a team's workgroups need not be resident together, and with a
    # short poll limit the waits that run long leave their teams to the repair launch.
    # Scores and centroids must equal those of a run on an otherwise idle GPU, bit for bit
    K, _, _ = synth.manifold_global(4, 1, 8, 16384, planted=8, seed=61, device=DEV)
    kvc_option("score_path", 1)
    G = K.shape[0]

    def score():
        mu = torch.empty((G, 128), dtype=torch.float32, device=DEV)
        return gpu_lib.kvc_score_l2(K, centroid=mu).clone(), mu

    ref, ref_mu = score()
    torch.cuda.synchronize()
    a = torch.randn(6144, 6144, device=DEV)
    b = torch.randn(6144, 6144, device=DEV)
    side = torch.cuda.Stream()  # default priority
    kvc_option("score_spin_limit", 256)
    outs = []
    for _ in range(3):
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for _ in range(4):
                c = a @ b
        outs.append(score())
    torch.cuda.synchronize()
    del c
    for sc, mu in outs:
        assert torch.equal(sc, ref) and torch.equal(mu, ref_mu)


def test_topk_ranks_nan_scores_below_every_number(gpu_lib):
    # order keys map NaN below -inf: with k no larger than the count of numbers in
    # every slice no NaN is kept, and the kept set is the top-k of the numbers
    G, S = 24, 5000
    s = synth.random_scores(G, S, seed=40, device=DEV)
    rng = np.random.default_rng(41)
    nan = torch.from_numpy(rng.random((G, S)) < 0.3).to(DEV)
    nan[:, :256] = True  # whole leading tile as well
    s = torch.where(nan, torch.full_like(s, float("nan")), s)
    k = int((~nan).sum(1).min())
    idx, _, _ = gpu_lib.kvc_topk_compact(s, k)
    assert not torch.gather(nan, 1, idx.long()).any()
    fin = torch.where(nan, torch.full_like(s, -1.0), s).cpu().numpy()  # the scores are >= 0
    np.testing.assert_array_equal(idx.cpu().numpy(), oracle.topk(fin, k))


def test_random_team_sizes_single_read_matches_three_launch_and_repair(gpu_lib, kvc_option):
    # 30 seeded shapes whose teams (slices or windows) have 33 to 700 tiles and often a
    # ragged last tile, global and windowed, L2 and cosine: the single-read kernel agrees
    # with the three-launch path (rel 1e-4) and, on the smaller ones, with the oracle;
    # a run whose every centroid wait gives up is repaired to the same bits
    rng = np.random.default_rng(2024)
    for _ in range(30):
        M = int(rng.choice([33, 40, 63, 65, 97, 129, 200, 257, 300, 385, 513, 700]))
        if rng.random() < 0.4:
            W = M * 256 - int(rng.integers(0, 255))
            S = int(W * rng.uniform(1.0, 3.5))
        else:
            S, W = M * 256 - int(rng.integers(0, 255)), None
        G = int(rng.integers(1, max(1, min(12, 1_500_000 // S)) + 1))
        metric = "cosine" if rng.random() < 0.3 else "l2"
        K, _, _ = synth.manifold_global(1, 1, G, S, planted=4, seed=int(rng.integers(1 << 30)), device=DEV)
        nwin = 1 if W is None else -(-S // W)

        def score(path, spin=-1):
            kvc_option("score_path", path)
            kvc_option("score_spin_limit", spin)
            mu = torch.empty((G, nwin, 128), dtype=torch.float32, device=DEV)
            return gpu_lib.kvc_score_centroid(K, W=W, metric=metric, centroids=mu).clone(), mu

        f, fmu = score(1)
        r, rmu = score(1, 0)
        u, _ = score(2)
        kvc_option("score_spin_limit", -1)
        torch.cuda.synchronize()
        case = (G, S, W, metric)
        assert not torch.isnan(f).any(), case
        assert torch.equal(f, r) and torch.equal(fmu, rmu), case
        rel = ((f - u).abs() / u.abs().clamp_min(1e-6)).max().item()
        assert rel < 1e-4, (rel, case)
        if metric == "l2" and G * S <= 400_000:
            _scores_vs_oracle(K, f, W)
