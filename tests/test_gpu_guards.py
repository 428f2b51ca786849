"""Guard regions around every output of the C ABI: each output buffer is taken from
a larger allocation filled with a canary pattern, so that a write past its end
(past G*S scores, past k kept rows, past the packed sum of the ragged budgets)
shows as a changed canary byte.  Where the ABI promises that rows t >= S of a
strided output stay unwritten, those rows are filled with the canary too and
checked.  Every input is seeded; the kernels run in the launch configurations
the entry points choose (the scoring kernel on both of its paths)."""
import numpy as np
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu
DEV = "cuda"
PAD = 4096  # guard bytes after every output
CANARY = 0xA5


class Guarded:
    """An output view of `shape` inside a canary-filled buffer with PAD guard bytes
    after it."""

    def __init__(self, shape, dtype):
        n = int(np.prod(shape)) * torch.tensor([], dtype=dtype).element_size()
        self.raw = torch.full((n + PAD,), CANARY, dtype=torch.uint8, device=DEV)
        self.n = n
        self.t = self.raw[:n].view(dtype).view(shape)

    def guard_intact(self):
        torch.cuda.synchronize()
        return bool(torch.all(self.raw[self.n:] == CANARY))

    def rows_intact(self, S):
        """Rows t >= S of a [G, S_stride, ...] output still hold the canary."""
        torch.cuda.synchronize()
        tail = self.t[:, S:].contiguous().view(torch.uint8)
        return bool(torch.all(tail == CANARY))


@pytest.mark.parametrize("path", [1, 2])
@pytest.mark.parametrize("W", [None, 1000])
def test_scoring_writes_nothing_past_its_outputs(gpu_lib, kvc_option, path, W):
    kvc_option("score_path", path)
    G, S = 24, 5000
    K, _, _ = synth.manifold_global(1, 1, G, S, planted=4, seed=31, device=DEV)
    nwin = 1 if W is None else -(-S // W)
    sc = Guarded((G, S), torch.float32)
    mu = Guarded((G, nwin, 128), torch.float32)
    gpu_lib.kvc_score_centroid(K, W=W, scores=sc.t, centroids=mu.t)
    assert sc.guard_intact() and mu.guard_intact()
    assert not torch.isnan(sc.t).any()


def test_topk_writes_nothing_past_k(gpu_lib, kvc_option):
    G, S, stride, k = 300, 3000, 3072, 1111
    s = synth.random_scores(G, stride, seed=32, device=DEV)
    K = torch.randint(-32768, 32767, (G, stride, 128), dtype=torch.int16, device=DEV).view(torch.bfloat16)
    V = torch.randint(-32768, 32767, (G, stride, 128), dtype=torch.int16, device=DEV).view(torch.bfloat16)
    for gather in (0, 1):  # the wide gather and the in-workgroup copy
        kvc_option("gather_path", gather)
        idx, Ko, Vo = (Guarded((G, k), torch.int32), Guarded((G, k, 128), torch.bfloat16),
                       Guarded((G, k, 128), torch.bfloat16))
        gpu_lib.kvc_topk_compact(s, k, K, V, S=S, idx_out=idx.t, K_out=Ko.t, V_out=Vo.t)
        assert idx.guard_intact() and Ko.guard_intact() and Vo.guard_intact()
        assert int(idx.t.max()) < S


def test_ragged_writes_nothing_past_the_packed_rows(gpu_lib):
    G, S = 40, 2000
    ks = np.random.default_rng(33).integers(0, S + 1, G)
    total = int(ks.sum())
    s = synth.random_scores(G, S, seed=34, device=DEV)
    K = torch.randint(-32768, 32767, (G, S, 128), dtype=torch.int16, device=DEV).view(torch.bfloat16)
    idx, Ko, Vo = (Guarded((total,), torch.int32), Guarded((total, 128), torch.bfloat16),
                   Guarded((total, 128), torch.bfloat16))
    gpu_lib.kvc_topk_compact_ragged(s, ks, K, K, idx_out=idx.t, K_out=Ko.t, V_out=Vo.t)
    gpu_lib.kvc_workspace_status()
    assert idx.guard_intact() and Ko.guard_intact() and Vo.guard_intact()


@pytest.mark.parametrize("R", [32, 64, 128])
@pytest.mark.parametrize("storage", ["fp32", "bf16"])
def test_lowrank_leaves_rows_past_S_and_the_guards(gpu_lib, R, storage):
    # strided cache (S_stride > S): rows t >= S of K~, V~, err, K^, V^ stay unwritten,
    # for the stand-alone compression, the reconstruction and the fused pass
    L, B, Hkv, Hq, S, stride, Wq = 2, 1, 2, 8, 1000, 1100, 4
    G = L * B * Hkv
    inp = synth.oja_inputs(L, B, Hkv, Hq, S, R=R, Wq=Wq, S_cap=stride, seed=35, device=DEV)
    dt = torch.bfloat16 if storage == "bf16" else torch.float32
    sfx = "_bf16" if storage == "bf16" else ""
    Kt, Vt, err = Guarded((G, stride, R), dt), Guarded((G, stride, R), dt), Guarded((G, stride), torch.float32)
    getattr(gpu_lib, "kvc_lowrank_compress" + sfx)(inp.K, inp.V, inp.Q, inp.Uk, inp.Uv, L, B, Hkv, S=S,
                                                   K_tilde=Kt.t, V_tilde=Vt.t, err=err.t)
    for o in (Kt, Vt, err):
        assert o.rows_intact(S) and o.guard_intact()
    k = 50
    idx, Ka, _ = gpu_lib.kvc_topk_compact(err.t, k, inp.K, inp.V, S=S)
    Kh = Guarded((G, stride, 128), dt)
    getattr(gpu_lib, "kvc_reconstruct" + sfx)(Kt.t, inp.Uk, idx, Ka, L, B, Hkv, S=S, X_hat=Kh.t)
    assert Kh.rows_intact(S) and Kh.guard_intact()
    if R <= 64:
        outs = [Guarded((G, stride, R), dt), Guarded((G, stride, R), dt), Guarded((G, stride), torch.float32),
                Guarded((G, stride, 128), dt), Guarded((G, stride, 128), dt)]
        getattr(gpu_lib, "kvc_lowrank_compress_reconstruct" + sfx)(
            inp.K, inp.V, inp.Q, inp.Uk, inp.Uv, L, B, Hkv, S=S, K_tilde=outs[0].t, V_tilde=outs[1].t,
            err=outs[2].t, K_hat=outs[3].t, V_hat=outs[4].t)
        getattr(gpu_lib, "kvc_place_anchors" + sfx)(idx, Ka, L, B, Hkv, outs[3].t, S=S)
        for o in outs:
            assert o.rows_intact(S) and o.guard_intact()


def test_oja_refine_and_append_guards(gpu_lib):
    L, B, Hkv, N, R = 2, 2, 3, 700, 64
    X = torch.randn((L * B * Hkv, N, 128), generator=torch.Generator().manual_seed(36)).to(torch.bfloat16).to(DEV)
    U = Guarded((L, Hkv, 128, R), torch.float32)
    U.t.copy_(torch.from_numpy(np.stack([[synth.orthonormal_basis(128, R, 36, l, h) for h in range(Hkv)]
                                         for l in range(L)])))
    gpu_lib.kvc_oja_update(U.t, X, 32, 1e-3, L, B, Hkv)
    assert U.guard_intact()
    G, S, c, nq = 6, 1234, 10, 4
    K, V, _ = synth.manifold_global(1, 1, G, S, planted=4, seed=37, device=DEV)
    mk, mv, rad, vn = gpu_lib.kvc_cluster_summaries(K, V, c)
    Q = torch.randn((G, nq, 128), generator=torch.Generator().manual_seed(38)).to(torch.bfloat16).to(DEV)
    rc = Guarded((G, nq, mk.shape[1]), torch.float32)
    gpu_lib.kvc_refine_risk(mk, rad, vn, S, c, Q, rc=rc.t)
    assert rc.guard_intact()
