"""GPU parity of retention with a budget per slice (kvc_topk_compact_ragged) driven
by RippleKV's layer budgets ("RippleKV: Cross-Layer KV Cache Allocation via
Perturbation Propagation", sensitivity-guided budget allocation: every slice of
layer l keeps k_l tokens, the token selector itself unchanged).  Index sets are
bit-exact on identical scores; rows bit-exact; end to end with ManifoldKV scores
the retained sets agree with the oracle's up to the threshold band."""
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import oracle
import synth
from tests.helpers import index_sets_agree

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _check_packed(idx, Ko, Vo, ks, s_host, Kb, Vb, S=None):
    ref = oracle.topk_ragged(s_host, ks, S)
    np.testing.assert_array_equal(idx.cpu().numpy(), ref)
    if Ko is not None:
        off = np.concatenate([[0], np.cumsum(ks)])
        ko, vo = synth.bf16_bits(Ko), synth.bf16_bits(Vo)
        for g in range(len(ks)):
            sel = ref[off[g]:off[g + 1]].astype(np.int64)
            np.testing.assert_array_equal(ko[off[g]:off[g + 1]], Kb[g][sel])
            np.testing.assert_array_equal(vo[off[g]:off[g + 1]], Vb[g][sel])


@pytest.mark.parametrize("separate", [False, True])
def test_ragged_layer_budgets_bit_exact(gpu_lib, kvc_option, separate):
    # 30 layers x 10 slices, S = 5000 with a ragged stride; budgets from a sensitivity
    # profile (some layers pinned at S, none empty) and ties in the scores
    kvc_option("gather_path", 0 if separate else 1)
    L, per, S, stride = 30, 10, 5000, 5003
    G = L * per
    rng = np.random.default_rng(21)
    kl = gpu_lib.kvc_layer_budgets(rng.exponential(1.0, L), 16.0, 4.0, L * S // 3, S)
    ks = np.repeat(kl, per)
    s = synth.random_scores(G, stride, seed=22, kind="ties", device="cpu")
    K = torch.randint(-32768, 32767, (G, stride, 128), dtype=torch.int16, device=DEV).view(torch.bfloat16)
    V = torch.randint(-32768, 32767, (G, stride, 128), dtype=torch.int16, device=DEV).view(torch.bfloat16)
    idx, Ko, Vo = gpu_lib.kvc_topk_compact_ragged(s.to(DEV), ks, K, V, S=S)
    torch.cuda.synchronize()
    _check_packed(idx, Ko, Vo, ks, s.numpy(), synth.bf16_bits(K), synth.bf16_bits(V), S)


def test_ragged_zero_full_and_large_budgets(gpu_lib):
    # budgets 0, 1, S and above the in-workgroup copy limit (8192), mixed
    G, S = 6, 20000
    ks = np.array([0, 1, S, 9000, 0, 12345])
    s = synth.random_scores(G, S, seed=23, device="cpu")
    K = torch.randint(-32768, 32767, (G, S, 128), dtype=torch.int16, device=DEV).view(torch.bfloat16)
    V = torch.randint(-32768, 32767, (G, S, 128), dtype=torch.int16, device=DEV).view(torch.bfloat16)
    idx, Ko, Vo = gpu_lib.kvc_topk_compact_ragged(s.to(DEV), ks, K, V)
    torch.cuda.synchronize()
    _check_packed(idx, Ko, Vo, ks, s.numpy(), synth.bf16_bits(K), synth.bf16_bits(V))
    idx2, _, _ = gpu_lib.kvc_topk_compact_ragged(s.to(DEV), ks)  # indices only
    torch.cuda.synchronize()
    assert torch.equal(idx, idx2)


def test_empty_selections_with_rows_given(gpu_lib):
    # nothing to keep (k = 0, or every budget 0): the empty outputs the binding passes
    # have no storage, and the calls succeed without writing anything
    G, S = 5, 700
    s = synth.random_scores(G, S, seed=31, device=DEV)
    K = torch.zeros((G, S, 128), dtype=torch.bfloat16, device=DEV)
    idx, Ko, Vo = gpu_lib.kvc_topk_compact(s, 0, K, K)
    assert idx.numel() == 0 and Ko.numel() == 0 and Vo.numel() == 0
    idx, Ko, Vo = gpu_lib.kvc_topk_compact_ragged(s, [0] * G, K, K)
    torch.cuda.synchronize()
    gpu_lib.kvc_workspace_status()
    assert idx.numel() == 0 and Ko.numel() == 0 and Vo.numel() == 0


def test_ragged_with_uniform_budgets_equals_topk(gpu_lib):
    G, S, k = 40, 3000, 777
    s = synth.random_scores(G, S, seed=24, device="cpu").to(DEV)
    a, _, _ = gpu_lib.kvc_topk_compact(s, k)
    b, _, _ = gpu_lib.kvc_topk_compact_ragged(s, [k] * G)
    torch.cuda.synchronize()
    assert torch.equal(a.view(-1), b)


def test_ripplekv_eviction_llama_shape(gpu_lib):
    # ManifoldKV scores on the 32-layer x 8-kv-head cache (S = 16384); per-layer budgets
    # from a seeded sensitivity profile, total 50% of the cache; every slice checked
    L, H, S = 32, 8, 16384
    K, V, _ = synth.manifold_global(L, 1, H, S, planted=64, device=DEV)
    sens = np.random.default_rng(25).gamma(2.0, 1.0, L)
    kl = gpu_lib.kvc_layer_budgets(sens, 8.0, 4.0, L * S // 2, S)
    assert kl.sum() == L * S // 2
    ks = np.repeat(kl, H)
    sc = gpu_lib.kvc_score_l2(K)
    idx, Ko, Vo = gpu_lib.kvc_topk_compact_ragged(sc, ks, K, V)
    torch.cuda.synchronize()
    kb, vb = synth.bf16_bits(K), synth.bf16_bits(V)
    idx_h, ko, vo = idx.cpu().numpy(), synth.bf16_bits(Ko), synth.bf16_bits(Vo)
    off = np.concatenate([[0], np.cumsum(ks)])

    def check(g):
        ora, _ = oracle.score_l2(kb[g:g + 1])
        o32 = ora.astype(np.float32)
        gi = idx_h[off[g]:off[g + 1]][None]
        ok, _ = index_sets_agree(gi, oracle.topk(o32, int(ks[g])), o32, int(ks[g]))
        assert ok, "slice %d" % g
        sel = gi[0].astype(np.int64)
        np.testing.assert_array_equal(ko[off[g]:off[g + 1]], kb[g][sel])
        np.testing.assert_array_equal(vo[off[g]:off[g + 1]], vb[g][sel])

    with ThreadPoolExecutor(max_workers=8) as ex:
        list(ex.map(check, range(L * H)))


def test_ragged_device_budgets_checked_on_device(gpu_lib):
    # budgets handed over as a device array: a budget above k_max, a negative one, and one
    # whose rows would end past the packed capacity k_total keep nothing (reported by the
    # status query), nothing is written outside [0, k_total), and every other slice is
    # exactly the oracle's selection at its offset
    G, S = 5, 3000
    s = synth.random_scores(G, S, seed=26, device="cpu")
    K = torch.randint(-32768, 32767, (G, S, 128), dtype=torch.int16, device=DEV).view(torch.bfloat16)
    ks = np.array([100, 2500, -3, 700, 400], dtype=np.int64)  # 2500 > k_max; -3 < 0
    k_max, k_total = 1000, 100 + 700 + 300  # slice 4's 400 rows do not fit after slice 3's
    pad = 64
    idx = torch.full((k_total + pad,), -7, dtype=torch.int32, device=DEV)
    Ko = torch.full((k_total + pad, 128), 0x1234, dtype=torch.int16, device=DEV).view(torch.bfloat16)
    kd = torch.from_numpy(ks).to(DEV)
    gpu_lib.kvc_topk_compact_ragged(s.to(DEV), kd, K, None, idx_out=idx[:k_total], K_out=Ko[:k_total],
                                    k_max=k_max, k_total=k_total)
    with pytest.raises(gpu_lib.KvcError) as err:
        gpu_lib.kvc_workspace_status()
    assert err.value.status == gpu_lib.ERR_INVALID_ARGUMENT
    ih = idx.cpu().numpy()
    kept = [(0, 100, 0), (3, 700, 100)]  # (slice, budget, offset) of the slices that fit
    for g, k, off in kept:
        np.testing.assert_array_equal(ih[off:off + k], oracle.topk(s[g:g + 1].numpy(), k)[0])
        np.testing.assert_array_equal(synth.bf16_bits(Ko[off:off + k]),
                                      synth.bf16_bits(K)[g][ih[off:off + k].astype(np.int64)])
    assert np.all(ih[800:] == -7)  # rows of the slice that did not fit and the guard stay untouched
    assert torch.all(Ko[800:].view(torch.int16) == 0x1234)
    # valid device budgets: the status query reports nothing
    kd2 = torch.from_numpy(np.array([100, 200, 0, 300, 400], dtype=np.int64)).to(DEV)
    a, _, _ = gpu_lib.kvc_topk_compact_ragged(s.to(DEV), kd2, k_max=400, k_total=1000)
    gpu_lib.kvc_workspace_status()
    np.testing.assert_array_equal(a.cpu().numpy(), oracle.topk_ragged(s.numpy(), [100, 200, 0, 300, 400]))
