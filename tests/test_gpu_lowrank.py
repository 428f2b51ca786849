"""GPU parity of the OjaKV hybrid low-rank path against the CPU oracle, through
the C ABI: projection K~/V~ and reconstruction within rel 2e-3 of
(|oracle| + rms(slice)); the error score e_t (an fp32 score) within rel 1e-4;
Oja/QR bases within rel 2e-3 and orthonormal to 1e-5; anchors by the
threshold-band rule; anchor rows exact."""
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import oracle
import synth
from tests.helpers import index_sets_agree, lowrank_close, score_close

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _compress_check(gpu_lib, inp, slices=None, S=None, threads=8):
    S = inp.S if S is None else S
    Kt, Vt, err = gpu_lib.kvc_lowrank_compress(inp.K, inp.V, inp.Q, inp.Uk, inp.Uv, inp.L, inp.B,
                                               inp.Hkv, S=S)
    torch.cuda.synchronize()
    G = inp.L * inp.B * inp.Hkv
    slices = list(range(G) if slices is None else slices)
    Uk = inp.Uk.cpu().numpy()
    Uv = inp.Uv.cpu().numpy()
    grp = inp.Hq // inp.Hkv
    host = {}
    for g in slices:  # device -> host copies stay on this thread
        l, b, h = g // (inp.B * inp.Hkv), (g // inp.Hkv) % inp.B, g % inp.Hkv
        host[g] = (synth.bf16_bits(inp.K[g:g + 1, :S]), synth.bf16_bits(inp.V[g:g + 1, :S]),
                   synth.bf16_bits(inp.Q[l:l + 1, b:b + 1, h * grp:(h + 1) * grp]),
                   Kt[g:g + 1, :S].cpu().numpy(), Vt[g:g + 1, :S].cpu().numpy(),
                   err[g:g + 1, :S].cpu().numpy())

    def check(g):
        l, h = g // (inp.B * inp.Hkv), g % inp.Hkv
        kb, vb, Q, kt, vt, eg = host[g]
        okt, ovt, oerr = oracle.lowrank_compress(kb, vb, Q, Uk[l:l + 1, h:h + 1], Uv[l:l + 1, h:h + 1],
                                                 1, 1, 1, grp)
        ok, rel = lowrank_close(kt, okt)
        assert ok, "K~ slice %d: max rel %.3g" % (g, rel)
        ok, rel = lowrank_close(vt, ovt)
        assert ok, "V~ slice %d: max rel %.3g" % (g, rel)
        ok, rel, nbad = score_close(eg, oerr)
        assert ok, "err slice %d: %d off, max rel %.3g" % (g, nbad, rel)
        return oerr

    # single-threaded C oracle through ctypes (GIL released): slices checked concurrently
    with ThreadPoolExecutor(max_workers=threads) as ex:
        oerrs = dict(zip(slices, ex.map(check, slices)))
    return Kt, Vt, err, oerrs


@pytest.mark.parametrize("R", [32, 64, 96, 128])
def test_compress_small(gpu_lib, R):
    inp = synth.oja_inputs(2, 2, 2, 8, 700, R=R, Wq=32, seed=R, device=DEV)
    _compress_check(gpu_lib, inp)


@pytest.mark.parametrize("Hq,Wq", [(2, 1), (4, 7), (16, 8), (12, 14)])
def test_compress_window_shapes(gpu_lib, Hq, Wq):
    # |W| = g*Wq of 1, 14, 64 and 84 queries (one to three 32-query blocks of the folded
    # query); ragged token tail; strided cache (S < S_stride)
    inp = synth.oja_inputs(1, 1, 2, Hq, 333, R=64, Wq=Wq, S_cap=400, seed=Hq * 100 + Wq, device=DEV)
    _compress_check(gpu_lib, inp, S=333)


def test_compress_without_query_or_values(gpu_lib):
    inp = synth.oja_inputs(1, 1, 2, 8, 300, R=64, Wq=4, device=DEV)
    Kt, Vt, err = gpu_lib.kvc_lowrank_compress(inp.K, None, None, inp.Uk, None, 1, 1, 2)
    torch.cuda.synchronize()
    assert Vt is None and err is None
    okt, _, _ = oracle.lowrank_compress(synth.bf16_bits(inp.K), None, None, inp.Uk.cpu().numpy(), None,
                                        1, 1, 2, 0)
    ok, rel = lowrank_close(Kt.cpu().numpy(), okt)
    assert ok, rel


def test_prefill_1024x32768_r64_every_slice(gpu_lib):
    # 32 layers x batch 4 x 8 kv heads x 32 query heads, S=32768, r=64, 32-query window,
    # 5% anchors, launched at full size (the OjaKV efficiency workload).  Every one of the
    # 1024 slices: e_t against the oracle (rel 1e-4), the anchor set by the threshold-band
    # rule and the anchor rows bit for bit; K~ and V~ on layers 0, 15 and 31 (96 slices).
    # The single-threaded oracle runs on 16 host threads; slices are copied to the host
    # in chunks on this thread.
    L, B, Hkv, Hq, S = 32, 4, 8, 32, 32768
    inp = synth.oja_inputs(L, B, Hkv, Hq, S, R=64, Wq=32, device=DEV)
    Kt, Vt, err = gpu_lib.kvc_lowrank_compress(inp.K, inp.V, inp.Q, inp.Uk, inp.Uv, L, B, Hkv)
    k = oracle.n_anchors(S)
    idx, Ka, Va = gpu_lib.kvc_topk_compact(err, k, inp.K, inp.V)
    torch.cuda.synchronize()
    Uk, Uv = inp.Uk.cpu().numpy(), inp.Uv.cpu().numpy()
    grp = Hq // Hkv
    full = {0, 15, 31}  # layers whose K~ and V~ are compared too

    def check(item):
        g, kb, vb, q, e_gpu, i_gpu, ka, va, kt, vt = item
        l, h = g // (B * Hkv), g % Hkv
        okt, ovt, oerr = oracle.lowrank_compress(kb, vb, q, Uk[l:l + 1, h:h + 1],
                                                 Uv[l:l + 1, h:h + 1] if vb is not None else None,
                                                 1, 1, 1, grp)
        ok, rel, nbad = score_close(e_gpu, oerr)
        assert ok, "err slice %d: %d off, max rel %.3g" % (g, nbad, rel)
        e32 = oerr.astype(np.float32)
        ok, _ = index_sets_agree(i_gpu, oracle.topk(e32, k), e32, k)
        assert ok, "anchors slice %d" % g
        sel = i_gpu[0].astype(np.int64)
        np.testing.assert_array_equal(ka, kb[0][sel])
        if kt is not None:
            np.testing.assert_array_equal(va, vb[0][sel])
            for got, want, name in ((kt, okt, "K~"), (vt, ovt, "V~")):
                ok, rel = lowrank_close(got, want)
                assert ok, "%s slice %d: max rel %.3g" % (name, g, rel)
        return g

    done = []
    chunk = 64
    with ThreadPoolExecutor(max_workers=16) as ex:
        for g0 in range(0, L * B * Hkv, chunk):
            items = []
            for g in range(g0, g0 + chunk):
                l, b, h = g // (B * Hkv), (g // Hkv) % B, g % Hkv
                with_v = l in full
                items.append((g, synth.bf16_bits(inp.K[g:g + 1]),
                              synth.bf16_bits(inp.V[g:g + 1]) if with_v else None,
                              synth.bf16_bits(inp.Q[l:l + 1, b:b + 1, h * grp:(h + 1) * grp]),
                              err[g:g + 1].cpu().numpy(), idx[g:g + 1].cpu().numpy(), synth.bf16_bits(Ka[g]),
                              synth.bf16_bits(Va[g]) if with_v else None,
                              Kt[g:g + 1].cpu().numpy() if with_v else None,
                              Vt[g:g + 1].cpu().numpy() if with_v else None))
            done += list(ex.map(check, items))
    assert done == list(range(L * B * Hkv))


@pytest.mark.parametrize("R,k", [(32, 0), (64, 17), (128, 5)])
def test_reconstruct_small(gpu_lib, R, k):
    L, B, Hkv, S = 2, 1, 3, 517
    G = L * B * Hkv
    Xt = synth.random_lowrank(G, S, R, seed=R).to(DEV)
    U = torch.from_numpy(np.stack([[synth.orthonormal_basis(128, R, 3, l, h) for h in range(Hkv)]
                                   for l in range(L)])).to(DEV)
    rng = np.random.default_rng(R + k)
    idx = np.sort(np.stack([rng.choice(S, k, replace=False) for _ in range(G)]), 1).astype(np.int32)
    rows = synth.bf16_bits(torch.randn((G, k, 128)).to(torch.bfloat16))
    idx_t = torch.from_numpy(idx).to(DEV) if k else None
    rows_t = synth.from_bits(rows, DEV) if k else None
    Xh = gpu_lib.kvc_reconstruct(Xt, U, idx_t, rows_t, L, B, Hkv)
    torch.cuda.synchronize()
    ora = oracle.reconstruct(Xt.cpu().numpy(), U.cpu().numpy(), idx if k else None, rows if k else None,
                             L, B, Hkv)
    ok, rel = lowrank_close(Xh.cpu().numpy(), ora)
    assert ok, rel
    for g in range(G):  # anchors exact
        np.testing.assert_array_equal(Xh[g].cpu().numpy()[idx[g]], ora[g][idx[g]])


@pytest.mark.parametrize("B,N,pool,eta,R", [(1, 4096, 32, 1e-3, 64), (2, 700, 7, 0.05, 64),
                                            (1, 32, 1, 1e-3, 64), (3, 64, 1, 0.1, 64),
                                            (1, 500, 4, 0.02, 32), (2, 64, 1, 0.1, 32), (2, 300, 3, 0.02, 96),
                                            (1, 256, 1, 0.02, 128)])
def test_oja_update_small(gpu_lib, B, N, pool, eta, R):
    # R <= 64 runs the LDS-resident step + QR, larger R the workspace-backed one
    L, Hkv = 2, 2
    inp = synth.oja_inputs(L, B, Hkv, 4, N, R=R, Wq=1, seed=N + B, device=DEV)
    U0 = inp.Uk.clone()
    U = inp.Uk.clone()
    gpu_lib.kvc_oja_update(U, inp.K, pool, eta, L, B, Hkv)
    torch.cuda.synchronize()
    ora = oracle.oja_update(U0.cpu().numpy(), synth.bf16_bits(inp.K), pool, eta, L, B, Hkv)
    Ug = U.cpu().numpy().astype(np.float64)
    ok, rel = lowrank_close(Ug.reshape(L * Hkv, -1), ora.reshape(L * Hkv, -1))
    assert ok, rel
    # the step itself (U' - U) is also matched, so the check is not carried by U alone;
    # at r = d the basis spans everything, C U - U U^T C U = 0 and the step is rounding noise
    if R < 128:
        d_gpu = Ug - U0.cpu().numpy()
        d_ora = ora - U0.cpu().numpy()
        ok, rel = lowrank_close(d_gpu.reshape(L * Hkv, -1), d_ora.reshape(L * Hkv, -1), rel=2e-3)
        assert ok, rel
    for l in range(L):
        for h in range(Hkv):
            assert np.abs(Ug[l, h].T @ Ug[l, h] - np.eye(R)).max() < 1e-5


def test_compress_determinism(gpu_lib):
    inp = synth.oja_inputs(1, 2, 4, 16, 3000, R=64, Wq=32, device=DEV)
    a = [t.clone() for t in gpu_lib.kvc_lowrank_compress(inp.K, inp.V, inp.Q, inp.Uk, inp.Uv, 1, 2, 4)]
    b = gpu_lib.kvc_lowrank_compress(inp.K, inp.V, inp.Q, inp.Uk, inp.Uv, 1, 2, 4)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_random_shapes_compress_and_fused_rebuild(gpu_lib):
    # 20 seeded shapes: ranks 32-128, 1-2 KV heads with 1, 2 or 4 query heads each, 1-32
    # window queries, odd lengths and strided caches, the fused reconstruction at ranks
    # <= 64 on about half -- K~, V~, e_t (and K^, V^) against the oracle
    rng = np.random.default_rng(77)
    for _ in range(20):
        R = int(rng.choice([32, 64, 96, 128]))
        Hkv, grp = int(rng.integers(1, 3)), int(rng.choice([1, 2, 4]))
        L, B = int(rng.integers(1, 3)), int(rng.integers(1, 3))
        S = int(rng.integers(1, 1500))
        Wq = int(rng.integers(1, 33))
        fused = R <= 64 and rng.random() < 0.5
        inp = synth.oja_inputs(L, B, Hkv, Hkv * grp, S, R=R, Wq=Wq, S_cap=S + int(rng.integers(0, 40)),
                               seed=int(rng.integers(1 << 30)), device=DEV)
        if fused:
            Kt, Vt, err, Kh, Vh = gpu_lib.kvc_lowrank_compress_reconstruct(inp.K, inp.V, inp.Q, inp.Uk, inp.Uv,
                                                                           L, B, Hkv, S=S)
        else:
            Kt, Vt, err = gpu_lib.kvc_lowrank_compress(inp.K, inp.V, inp.Q, inp.Uk, inp.Uv, L, B, Hkv, S=S)
        torch.cuda.synchronize()
        Uk, Uv = inp.Uk.cpu().numpy(), inp.Uv.cpu().numpy()
        case = (R, Hkv, grp, L, B, S, Wq, fused)
        for g in range(L * B * Hkv):
            l, b, h = g // (B * Hkv), (g // Hkv) % B, g % Hkv
            Q = synth.bf16_bits(inp.Q[l:l + 1, b:b + 1, h * grp:(h + 1) * grp])
            okt, ovt, oerr = oracle.lowrank_compress(synth.bf16_bits(inp.K[g:g + 1, :S]),
                                                     synth.bf16_bits(inp.V[g:g + 1, :S]), Q,
                                                     Uk[l:l + 1, h:h + 1], Uv[l:l + 1, h:h + 1], 1, 1, 1, grp)
            pairs = [(Kt, okt), (Vt, ovt)]
            if fused:
                pairs += [(Kh, oracle.reconstruct(okt, Uk[l:l + 1, h:h + 1], None, None, 1, 1, 1)),
                          (Vh, oracle.reconstruct(ovt, Uv[l:l + 1, h:h + 1], None, None, 1, 1, 1))]
            for gpu, ora in pairs:
                ok, rel = lowrank_close(gpu[g:g + 1, :S].cpu().numpy(), ora)
                assert ok, (rel, g, case)
            ok, rel, nbad = score_close(err[g:g + 1, :S].cpu().numpy(), oerr)
            assert ok, (rel, nbad, g, case)
