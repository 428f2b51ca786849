"""GPU parity of the bf16-storage variants of the hybrid low-rank cache
(kvc_lowrank_compress_bf16, kvc_reconstruct_bf16: the memory-saving layout of the
OjaKV efficiency analysis) and of eviction composed with low-rank compression
("OjaKV: Context-Aware Online Low-Rank KV Cache Compression", appendix A.9: token
selection and feature projection commute).  Rules: bf16 outputs within +-1 bf16
ulp of the oracle's value rounded to bf16 (an absolute floor of 1e-5 rms for
values near zero); the bf16 result is the nearest-even rounding of the fp32
path's result, bit for bit; composition is bit-exact."""
import numpy as np
import pytest
import torch

import oracle
import synth
from tests.helpers import bf16_close, bf16_bits_rne, score_close

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _bits(t):
    return synth.bf16_bits(t)


@pytest.mark.parametrize("R", [32, 64, 96, 128])
def test_compress_bf16_vs_oracle_and_fp32(gpu_lib, R):
    inp = synth.oja_inputs(2, 2, 2, 8, 700, R=R, Wq=32, seed=R + 5, device=DEV)
    Kb, Vb, eb = gpu_lib.kvc_lowrank_compress_bf16(inp.K, inp.V, inp.Q, inp.Uk, inp.Uv, inp.L, inp.B, inp.Hkv)
    Kf, Vf, ef = gpu_lib.kvc_lowrank_compress(inp.K, inp.V, inp.Q, inp.Uk, inp.Uv, inp.L, inp.B, inp.Hkv)
    torch.cuda.synchronize()
    # the bf16 outputs are the nearest-even rounding of the fp32 path's results
    np.testing.assert_array_equal(_bits(Kb), bf16_bits_rne(Kf.cpu().numpy()))
    np.testing.assert_array_equal(_bits(Vb), bf16_bits_rne(Vf.cpu().numpy()))
    assert torch.equal(eb, ef)
    G, grp = inp.L * inp.B * inp.Hkv, inp.Hq // inp.Hkv
    Uk, Uv = inp.Uk.cpu().numpy(), inp.Uv.cpu().numpy()
    for g in range(G):
        l, b, h = g // (inp.B * inp.Hkv), (g // inp.Hkv) % inp.B, g % inp.Hkv
        Q = _bits(inp.Q[l:l + 1, b:b + 1, h * grp:(h + 1) * grp])
        okt, ovt, oerr = oracle.lowrank_compress(_bits(inp.K[g:g + 1]), _bits(inp.V[g:g + 1]), Q,
                                                 Uk[l:l + 1, h:h + 1], Uv[l:l + 1, h:h + 1], 1, 1, 1, grp)
        ok, ulp = bf16_close(_bits(Kb[g:g + 1]), okt)
        assert ok, "K~ slice %d: %d ulps" % (g, ulp)
        ok, ulp = bf16_close(_bits(Vb[g:g + 1]), ovt)
        assert ok, "V~ slice %d: %d ulps" % (g, ulp)
        ok, rel, nbad = score_close(eb[g:g + 1].cpu().numpy(), oerr)
        assert ok, (g, rel, nbad)


def test_compress_bf16_strided_ragged(gpu_lib):
    inp = synth.oja_inputs(1, 1, 2, 4, 333, R=64, Wq=7, S_cap=400, seed=71, device=DEV)
    Kb, Vb, _ = gpu_lib.kvc_lowrank_compress_bf16(inp.K, inp.V, inp.Q, inp.Uk, inp.Uv, 1, 1, 2, S=333)
    Kf, Vf, _ = gpu_lib.kvc_lowrank_compress(inp.K, inp.V, inp.Q, inp.Uk, inp.Uv, 1, 1, 2, S=333)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(_bits(Kb[:, :333]), bf16_bits_rne(Kf[:, :333].cpu().numpy()))
    np.testing.assert_array_equal(_bits(Vb[:, :333]), bf16_bits_rne(Vf[:, :333].cpu().numpy()))


@pytest.mark.parametrize("R,k", [(32, 0), (64, 17), (96, 3), (128, 5)])
def test_reconstruct_bf16_vs_oracle(gpu_lib, R, k):
    L, B, Hkv, S = 2, 1, 3, 517
    G = L * B * Hkv
    Xt = synth.random_lowrank(G, S, R, seed=R + 1).to(torch.bfloat16).to(DEV)
    U = torch.from_numpy(np.stack([[synth.orthonormal_basis(128, R, 5, l, h) for h in range(Hkv)]
                                   for l in range(L)])).to(DEV)
    rng = np.random.default_rng(R * 3 + k)
    idx = np.sort(np.stack([rng.choice(S, k, replace=False) for _ in range(G)]), 1).astype(np.int32)
    rows = _bits(torch.randn((G, k, 128)).to(torch.bfloat16))
    idx_t = torch.from_numpy(idx).to(DEV) if k else None
    rows_t = synth.from_bits(rows, DEV) if k else None
    Xh = gpu_lib.kvc_reconstruct_bf16(Xt, U, idx_t, rows_t, L, B, Hkv)
    torch.cuda.synchronize()
    # the oracle reconstructs from the same bf16 X~ (an input here), widened exactly
    ora = oracle.reconstruct(Xt.float().cpu().numpy(), U.cpu().numpy(), idx if k else None,
                             rows if k else None, L, B, Hkv)
    gb = _bits(Xh)
    ok, ulp = bf16_close(gb, ora)
    assert ok, "X^ off by %d bf16 ulps" % ulp
    for g in range(G):  # anchors bit for bit
        np.testing.assert_array_equal(gb[g][idx[g]], rows[g])


@pytest.mark.parametrize("bf16", [False, True])
def test_eviction_then_lowrank_commutes(gpu_lib, bf16):
    # evict with ManifoldKV, then compress the retained rows, equals compressing the whole
    # cache and keeping the same rows: projection and error score are per token
    inp = synth.oja_inputs(2, 1, 4, 16, 3000, R=64, Wq=8, seed=13, device=DEV)
    G = inp.L * inp.B * inp.Hkv
    keep = 1500
    s = gpu_lib.kvc_score_l2(inp.K)
    idx, Kk, Vk = gpu_lib.kvc_topk_compact(s, keep, inp.K, inp.V)
    comp = gpu_lib.kvc_lowrank_compress_bf16 if bf16 else gpu_lib.kvc_lowrank_compress
    Kt_kept, Vt_kept, e_kept = comp(Kk, Vk, inp.Q, inp.Uk, inp.Uv, inp.L, inp.B, inp.Hkv)
    Kt_all, Vt_all, e_all = comp(inp.K, inp.V, inp.Q, inp.Uk, inp.Uv, inp.L, inp.B, inp.Hkv)
    torch.cuda.synchronize()
    ix = idx.long()
    for a, b in ((Kt_kept, Kt_all), (Vt_kept, Vt_all)):
        sel = torch.gather(b, 1, ix[:, :, None].expand(G, keep, b.shape[-1]))
        assert torch.equal(a.view(torch.int16) if bf16 else a, sel.view(torch.int16) if bf16 else sel)
    assert torch.equal(e_kept, torch.gather(e_all, 1, ix))


def test_compress_bf16_prefill_shape_sampled(gpu_lib):
    # 32 layers x batch 4 x 8 kv heads, S=32768, r=64, 128-query window; sampled slices
    inp = synth.oja_inputs(32, 4, 8, 32, 32768, R=64, Wq=32, device=DEV)
    Kb, Vb, eb = gpu_lib.kvc_lowrank_compress_bf16(inp.K, inp.V, inp.Q, inp.Uk, inp.Uv, 32, 4, 8)
    torch.cuda.synchronize()
    Uk, Uv = inp.Uk.cpu().numpy(), inp.Uv.cpu().numpy()
    for g in (0, 517, 1023):
        l, b, h = g // 32, (g // 8) % 4, g % 8
        Q = _bits(inp.Q[l:l + 1, b:b + 1, 4 * h:4 * h + 4])
        okt, ovt, oerr = oracle.lowrank_compress(_bits(inp.K[g:g + 1]), _bits(inp.V[g:g + 1]), Q,
                                                 Uk[l:l + 1, h:h + 1], Uv[l:l + 1, h:h + 1], 1, 1, 1, 4)
        for name, gb, o in (("K~", Kb, okt), ("V~", Vb, ovt)):
            ok, ulp = bf16_close(_bits(gb[g:g + 1]), o)
            assert ok, "%s slice %d: %d ulps" % (name, g, ulp)
        assert score_close(eb[g:g + 1].cpu().numpy(), oerr)[0]
