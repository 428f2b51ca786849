"""GPU parity of the OjaKV prefill + decode loop (appendix A.1 of the OjaKV
deep-notes page) against the oracle's loop, run independently on the same
inputs: after the prefill and after every decode update the bases (rel 2e-3,
orthonormal to 1e-5), error scores (rel 1e-4), anchor sets (threshold band)
and reconstructions (rel 2e-3, anchor rows exact) agree.

The loop's decode-time re-projection and re-selection over the whole cache is
the reading adopted for the full-loop workload (parity unpinned relative to
the pages); both sides implement that same reading."""
import threading

import numpy as np
import pytest
import torch

import oracle
import synth
from tests.helpers import index_sets_agree, lowrank_close, score_close
from token_scoring_eviction_amd import pipeline

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _run_gpu_loop(inp, steps, T, pool, eta, slices, token_sample=None):
    """Runs the loop on the GPU; snapshots the sampled slices after the prefill
    and each update.  Returns (snapshots, decode queries per step on host)."""
    L, B, Hkv = inp.L, inp.B, inp.Hkv
    Uk, Uv = inp.Uk.clone(), inp.Uv.clone()
    snaps = []
    qdec = []

    def snap(st):
        torch.cuda.synchronize()
        S = st.S
        k = pipeline.anchor_count(S)
        G = inp.L * inp.B * inp.Hkv
        idx = st.hybrid.idx.view(-1)[:G * k].view(G, k)
        out = {"S": S}
        for g in slices:
            l, h = g // (B * Hkv), g % Hkv
            rows = np.arange(S) if token_sample is None else np.unique(
                np.concatenate([token_sample(S), idx[g].cpu().numpy()]))
            rt = torch.from_numpy(rows).to(DEV)
            out[g] = dict(Uk=st.U_k[l, h].cpu().numpy(), Uv=st.U_v[l, h].cpu().numpy(),
                          err=st.hybrid.err[g, :S].cpu().numpy(), idx=idx[g].cpu().numpy(),
                          rows=rows, Khat=st.hybrid.Khat[g][rt].cpu().numpy(),
                          Vhat=st.hybrid.Vhat[g][rt].cpu().numpy())
        snaps.append(out)

    st = pipeline.ojakv_prefill(inp.K, inp.V, inp.Q, Uk, Uv, L, B, Hkv, inp.S, T=T, pool=pool, eta=eta)
    snap(st)
    for step in range(steps):
        k, v, q = synth.decode_token(inp, step)
        qdec.append(q.cpu())
        if pipeline.ojakv_decode_step(st, inp.K, inp.V, k, v, q, L, B, Hkv, T=T, eta=eta):
            snap(st)
    torch.cuda.synchronize()
    return snaps, torch.stack(qdec) if qdec else None


def _oracle_loop(inp, g, steps, T, pool, eta, qdec):
    l, b, h = g // (inp.B * inp.Hkv), (g // inp.Hkv) % inp.B, g % inp.Hkv
    grp = inp.Hq // inp.Hkv
    S_end = inp.S + steps
    K = synth.bf16_bits(inp.K[g, :S_end])
    V = synth.bf16_bits(inp.V[g, :S_end])
    Qp = synth.bf16_bits(inp.Q[l, b, h * grp:(h + 1) * grp])
    Qd = synth.bf16_bits(qdec[:, l, b, h * grp:(h + 1) * grp].to(torch.bfloat16)) if steps else \
        np.zeros((0, grp, inp.D), np.uint16)
    return oracle.full_loop_slice(K, V, Qp, Qd, inp.Uk[l, h].cpu().numpy(), inp.Uv[l, h].cpu().numpy(),
                                  inp.S, steps, T, pool, eta)


def _compare(snap_g, ora, S):
    for key in ("Uk", "Uv"):
        ok, rel = lowrank_close(snap_g[key][None], ora[key][None].astype(np.float64))
        assert ok, "%s rel %.3g" % (key, rel)
        U = snap_g[key].astype(np.float64)
        assert np.abs(U.T @ U - np.eye(U.shape[1])).max() < 1e-5
    ok, rel, nbad = score_close(snap_g["err"][None], ora["err"])
    assert ok, "err: %d off, max rel %.3g" % (nbad, rel)
    k = pipeline.anchor_count(S)
    e32 = ora["err"].astype(np.float32)
    ok, nb = index_sets_agree(snap_g["idx"][None], ora["idx"], e32, k)
    assert ok, "anchor sets differ beyond the threshold band"
    both = np.intersect1d(snap_g["idx"], ora["idx"][0])
    gpu_anchor = np.isin(snap_g["rows"], snap_g["idx"])
    ora_anchor = np.isin(snap_g["rows"], ora["idx"][0])
    same = gpu_anchor == ora_anchor
    for key in ("Khat", "Vhat"):
        ref = ora[key][0][snap_g["rows"]]
        ok, rel = lowrank_close(snap_g[key][same][None], ref[same][None])
        assert ok, "%s rel %.3g" % (key, rel)
    assert both.size >= k - nb


def test_loop_small_all_slices(gpu_lib):
    # 1 layer, 2 kv heads / 8 query heads, 4096-token prompt, 256 decode steps, T=32 -> 8 updates
    inp = synth.oja_inputs(1, 1, 2, 8, 4096, R=64, Wq=32, S_cap=4096 + 256, seed=41, device=DEV)
    snaps, qdec = _run_gpu_loop(inp, 256, 32, 32, 1e-3, slices=[0, 1])
    assert [s["S"] for s in snaps] == [4096 + 32 * j for j in range(9)]
    for g in (0, 1):
        res = _oracle_loop(inp, g, 256, 32, 32, 1e-3, qdec)
        for j, ora in enumerate(res):
            _compare(snaps[j][g], ora, ora["S"])


def test_loop_256x131072_every_update(gpu_lib):
    # 32 layers x batch 1 x 8 kv heads (32 query heads), 131072-token prompt pooled by 32 for
    # the prefill update, eta 1e-3, 256 decode steps with an update every 32, all at full
    # size on the GPU.  One slice in each of layers 0, 15 and 31 is compared with an
    # independent oracle run of the whole loop after the prefill and after every one of
    # the 8 updates (bases, error scores, anchor sets, K^/V^ on 4096 sampled tokens plus
    # the anchors).  The three oracle loops run on their own threads; each phase is
    # compared as soon as the oracle reaches it and its arrays are then dropped.
    S0, steps, T = 131072, 256, 32
    inp = synth.oja_inputs(32, 1, 8, 32, S0, R=64, Wq=32, S_cap=S0 + steps, device=DEV)
    sl = [3, 15 * 8 + 7, 31 * 8 + 0]  # (layer 0, kv head 3), (15, 7), (31, 0)
    rng = np.random.default_rng(0)
    snaps, qdec = _run_gpu_loop(inp, steps, T, 32, 1e-3, slices=sl,
                                token_sample=lambda S: np.sort(rng.choice(S, 4096, replace=False)))
    assert len(snaps) == 9 and snaps[-1]["S"] == S0 + steps
    checked = {g: [] for g in sl}
    errors = []

    def prepare(g):
        def on_update(j, st):
            try:
                _compare(snaps[j][g], st, st["S"])
                checked[g].append(j)
            except AssertionError as e:  # reported on the main thread
                errors.append("slice %d, phase %d: %s" % (g, j, e))
            for key in ("Kt", "Vt", "Khat", "Vhat"):
                st.pop(key, None)
        l, b, h = g // (inp.B * inp.Hkv), (g // inp.Hkv) % inp.B, g % inp.Hkv
        grp = inp.Hq // inp.Hkv
        K = synth.bf16_bits(inp.K[g, :S0 + steps])
        V = synth.bf16_bits(inp.V[g, :S0 + steps])
        Qp = synth.bf16_bits(inp.Q[l, b, h * grp:(h + 1) * grp])
        Qd = synth.bf16_bits(qdec[:, l, b, h * grp:(h + 1) * grp].to(torch.bfloat16))
        return K, V, Qp, Qd, inp.Uk[l, h].cpu().numpy(), inp.Uv[l, h].cpu().numpy(), on_update

    args = {g: prepare(g) for g in sl}  # host copies on this thread
    threads = [threading.Thread(target=lambda g=g: oracle.full_loop_slice(
        *args[g][:6], S0, steps, T, 32, 1e-3, on_update=args[g][6])) for g in sl]
    for th in threads:
        th.start()
    for th in threads:
        th.join()
    assert not errors, errors
    assert all(checked[g] == list(range(9)) for g in sl), checked


def test_decode_append_places_rows(gpu_lib):
    # one decode step's rows land bit for bit in the cache, the update buffer and the
    # query window (method details / A.1), and nothing else changes
    L, B, Hkv, Hq, S_cap, T, D = 2, 1, 3, 12, 50, 8, 128
    G = L * B * Hkv
    gen = torch.Generator().manual_seed(3)
    K = torch.randn((G, S_cap, D), generator=gen).to(torch.bfloat16).to(DEV)
    V = torch.randn((G, S_cap, D), generator=gen).to(torch.bfloat16).to(DEV)
    Kb = torch.randn((G, T, D), generator=gen).to(torch.bfloat16).to(DEV)
    Vb = torch.randn((G, T, D), generator=gen).to(torch.bfloat16).to(DEV)
    Qb = torch.randn((L, B, Hq, T, D), generator=gen).to(torch.bfloat16).to(DEV)
    k = torch.randn((G, D), generator=gen).to(torch.bfloat16).to(DEV)
    v = torch.randn((G, D), generator=gen).to(torch.bfloat16).to(DEV)
    q = torch.randn((L, B, Hq, D), generator=gen).to(torch.bfloat16).to(DEV)
    ref = [t.clone() for t in (K, V, Kb, Vb, Qb)]
    ref[0][:, 37] = k
    ref[1][:, 37] = v
    ref[2][:, 5] = k
    ref[3][:, 5] = v
    ref[4][:, :, :, 5] = q
    gpu_lib.kvc_decode_append(K, V, k, v, 37, L, B, Hkv, K_buf=Kb, V_buf=Vb, slot=5, q_new=q, Q_buf=Qb)
    torch.cuda.synchronize()
    for got, want in zip((K, V, Kb, Vb, Qb), ref):
        assert torch.equal(got.view(torch.int16), want.view(torch.int16))
    with pytest.raises(gpu_lib.KvcError):
        gpu_lib.kvc_decode_append(K, V, k, v, S_cap, L, B, Hkv)  # position past the capacity
