"""GPU parity of the RefineKV cluster summaries and risk scores ("RefineKV"
project page: "Summarize", "Select", Figure 2 formula) against the CPU oracle:
means rel 1e-5, radii / value norms / risk scores within the score rule (rel 1e-4
+ 1e-6 rms).  The risk kernel is checked on summaries given as inputs to both
sides, and end to end from K, V."""
import numpy as np
import pytest
import torch

import oracle
import synth
from tests.helpers import score_close

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.mark.parametrize("S,c", [(1000, 10), (4096, 32), (777, 50), (300, 1), (100, 1000), (5000, 257)])
def test_summaries_vs_oracle(gpu_lib, S, c):
    K, V, _ = synth.manifold_global(1, 1, 3, S, planted=min(4, S), seed=S + c, device=DEV)
    mk, mv, rad, vn = gpu_lib.kvc_cluster_summaries(K, V, c)
    torch.cuda.synchronize()
    omk, omv, orad, ovn = oracle.cluster_summaries(synth.bf16_bits(K), synth.bf16_bits(V), c)
    np.testing.assert_allclose(mk.cpu().numpy(), omk, rtol=1e-5, atol=1e-5)
    np.testing.assert_allclose(mv.cpu().numpy(), omv, rtol=1e-5, atol=1e-5)
    for got, ref in ((rad, orad), (vn, ovn)):
        ok, rel, nbad = score_close(got.cpu().numpy(), ref)
        assert ok, (rel, nbad)


@pytest.mark.parametrize("S,c", [(2000, 10), (100, 1000), (5000, 1), (262144 + 7, 33)])
@pytest.mark.parametrize("rmax", [4.0, 400.0])
@pytest.mark.parametrize("nq", [1, 4, 8])
def test_risk_on_given_summaries(gpu_lib, nq, rmax, S, c):
    # identical fp32 summaries and bf16 queries on both sides; radii up to 400 put
    # d_C = ||q|| radius / sqrt(D) far past where cosh overflows fp32 (d ~ 89).  Cluster
    # counts 200, 1 (a single short cluster), 5000 and 7944 (a short last cluster): one
    # or many 128-cluster chunks, one or several 2048-cluster final blocks, ragged tails
    G = 3
    nC = -(-S // c)
    rng = np.random.default_rng(nq)
    mk = rng.normal(0.0, 1.0, (G, nC, 128)).astype(np.float32)
    rad = rng.uniform(0.0, rmax, (G, nC)).astype(np.float32)
    vn = rng.uniform(5.0, 20.0, (G, nC)).astype(np.float32)
    Q = torch.from_numpy(rng.normal(0.0, 1.0, (G, nq, 128))).to(torch.bfloat16)
    rc = gpu_lib.kvc_refine_risk(torch.from_numpy(mk).to(DEV), torch.from_numpy(rad).to(DEV),
                                 torch.from_numpy(vn).to(DEV), S, c, Q.to(DEV))
    torch.cuda.synchronize()
    ora = oracle.refine_risk(mk, rad, vn, S, c, synth.bf16_bits(Q))
    for g in range(G):
        ok, rel, nbad = score_close(rc[g].cpu().numpy(), ora[g])
        assert ok, "slice %d: %d off, max rel %.3g" % (g, nbad, rel)


def test_refine_end_to_end_llama_layer(gpu_lib):
    # one layer of the 131072-token cache (8 kv heads), clusters of 10 keys (Figure 2), the
    # 4 query heads of each kv head; oracle from K, V, Q independently
    S, c = 131072, 10
    K, V, _ = synth.manifold_global(1, 1, 8, S, planted=64, seed=77, device=DEV)
    Q = torch.randn((8, 4, 128), generator=torch.Generator().manual_seed(5)).to(torch.bfloat16)
    mk, mv, rad, vn = gpu_lib.kvc_cluster_summaries(K, V, c)
    rc = gpu_lib.kvc_refine_risk(mk, rad, vn, S, c, Q.to(DEV))
    torch.cuda.synchronize()
    for g in (0, 5):
        omk, _, orad, ovn = oracle.cluster_summaries(synth.bf16_bits(K[g:g + 1]), synth.bf16_bits(V[g:g + 1]), c)
        ora = oracle.refine_risk(omk, orad, ovn, S, c, synth.bf16_bits(Q[g:g + 1]))
        ok, rel, nbad = score_close(rc[g].cpu().numpy(), ora[0])
        assert ok, "slice %d: %d off, max rel %.3g" % (g, nbad, rel)


def test_refine_bench_shape_sampled(gpu_lib):
    # the launch configuration the bench times: 32 layers x 8 kv heads x 131072 tokens,
    # 10-key clusters, 4 queries per kv head; three slices checked against the oracle
    L, H, S, c = 32, 8, 131072, 10
    K, V, _ = synth.manifold_global(L, 1, H, S, planted=64, seed=79, device=DEV)
    Q = torch.randn((L * H, 4, 128), generator=torch.Generator().manual_seed(6)).to(torch.bfloat16)
    mk, mv, rad, vn = gpu_lib.kvc_cluster_summaries(K, V, c)
    rc = gpu_lib.kvc_refine_risk(mk, rad, vn, S, c, Q.to(DEV))
    rc2 = gpu_lib.kvc_refine_risk(mk, rad, vn, S, c, Q.to(DEV))
    torch.cuda.synchronize()
    assert torch.equal(rc, rc2)  # the chunk records merge in a fixed order: bit-reproducible
    for g in (0, 137, 255):
        omk, omv, orad, ovn = oracle.cluster_summaries(synth.bf16_bits(K[g:g + 1]), synth.bf16_bits(V[g:g + 1]), c)
        np.testing.assert_allclose(mk[g].cpu().numpy(), omk[0], rtol=1e-5, atol=1e-5)
        np.testing.assert_allclose(mv[g].cpu().numpy(), omv[0], rtol=1e-5, atol=1e-5)
        for got, ref in ((rad, orad), (vn, ovn)):
            ok, rel, nbad = score_close(got[g:g + 1].cpu().numpy(), ref)
            assert ok, (g, rel, nbad)
        ora = oracle.refine_risk(omk, orad, ovn, S, c, synth.bf16_bits(Q[g:g + 1]))
        ok, rel, nbad = score_close(rc[g].cpu().numpy(), ora[0])
        assert ok, "slice %d: %d off, max rel %.3g" % (g, nbad, rel)
