"""Host orchestration of the C-ABI calls into the two hot paths (no arithmetic
here: every step runs in libkvc's HIP kernels).

* ManifoldKV eviction ("ManifoldKV: Training-Free KV Cache Compression via
  Euclidean Outlier Detection", abstract): score every key by its distance to
  the (global or windowed) key centroid, keep the `keep` farthest per slice,
  compact K and V to the kept rows.
* OjaKV hybrid low-rank loop ("OjaKV: Context-Aware Online Low-Rank KV Cache
  Compression", method details and appendix A.1): prefill pooled Oja update +
  QR, projection, error score, top-k full-rank anchors, reconstruction; then
  decode steps buffered T at a time, each full buffer triggering an unpooled
  update, re-projection of the whole cache, re-scoring, re-selection of
  anchors and reconstruction.
"""
from __future__ import annotations

from dataclasses import dataclass

import torch

from . import kvc


@dataclass
class EvictionBuffers:
    scores: torch.Tensor
    idx: torch.Tensor
    K_out: torch.Tensor
    V_out: torch.Tensor


def alloc_eviction(G, S, keep, D=128, device="cuda"):
    return EvictionBuffers(
        scores=torch.empty((G, S), dtype=torch.float32, device=device),
        idx=torch.empty((G, keep), dtype=torch.int32, device=device),
        K_out=torch.empty((G, keep, D), dtype=torch.bfloat16, device=device),
        V_out=torch.empty((G, keep, D), dtype=torch.bfloat16, device=device))


def manifold_evict(K, V, keep, W=None, buf: EvictionBuffers | None = None, metric="l2"):
    """One ManifoldKV eviction pass over K, V (bf16 [G, S, 128]).  W=None: global
    centroid; otherwise contiguous windows of W tokens.  metric "cosine" scores
    1 - cos(k, mu) instead of ||k - mu|| (the cosine-to-centroid baseline).
    Returns the buffers."""
    G, S, D = K.shape
    buf = buf or alloc_eviction(G, S, keep, D, K.device)
    if metric != "l2":
        kvc.kvc_score_centroid(K, W=W, metric=metric, scores=buf.scores)
    elif W is None:
        kvc.kvc_score_l2(K, scores=buf.scores)
    else:
        kvc.kvc_score_l2_windowed(K, W, scores=buf.scores)
    kvc.kvc_topk_compact(buf.scores, keep, K, V, idx_out=buf.idx, K_out=buf.K_out, V_out=buf.V_out)
    return buf


def anchor_count(S, percent=5):
    """ceil(percent * S / 100) full-rank anchors."""
    return -(-percent * S // 100)


@dataclass
class HybridState:
    """Hybrid cache of one OjaKV pass: K~/V~ for every token, the anchors'
    indices and full-rank rows, the error scores and the reconstruction."""
    Kt: torch.Tensor
    Vt: torch.Tensor
    err: torch.Tensor
    idx: torch.Tensor
    K_anchor: torch.Tensor
    V_anchor: torch.Tensor
    Khat: torch.Tensor
    Vhat: torch.Tensor


def alloc_hybrid(G, S_cap, R, D=128, device="cuda", max_anchor=None, with_hat=True, storage="fp32"):
    """storage "fp32": K~, V~, K^, V^ in fp32; "bf16": all four in bf16 (the
    memory-saving layout).  Error scores are fp32 either way."""
    max_anchor = anchor_count(S_cap) if max_anchor is None else max_anchor
    st = dict(dtype=torch.bfloat16 if storage == "bf16" else torch.float32, device=device)
    return HybridState(
        Kt=torch.empty((G, S_cap, R), **st), Vt=torch.empty((G, S_cap, R), **st),
        err=torch.empty((G, S_cap), dtype=torch.float32, device=device),
        idx=torch.empty((G, max_anchor), dtype=torch.int32, device=device),
        K_anchor=torch.empty((G, max_anchor, D), dtype=torch.bfloat16, device=device),
        V_anchor=torch.empty((G, max_anchor, D), dtype=torch.bfloat16, device=device),
        Khat=torch.empty((G, S_cap, D), **st) if with_hat else None,
        Vhat=torch.empty((G, S_cap, D), **st) if with_hat else None)


def hybrid_pass(K, V, Q_win, U_k, U_v, L, B, H_kv, S, st: HybridState, anchor_percent=5,
                reconstruct=True, fused=True):
    """Compress all S tokens, score them, keep ceil(p%) anchors at full rank and
    (optionally) rebuild K^, V^.  K, V: bf16 [G, S_cap, 128] caches (S <= S_cap).
    fused: K^, V^ come out of the compression launch (X~ is not read back) and
    only the anchor rows are written afterwards; the result is the same, bit
    for bit, as compress -> select -> reconstruct."""
    G = K.shape[0]
    k = anchor_count(S, anchor_percent)
    if k > st.idx.shape[1]:
        raise ValueError("anchor buffers hold %d rows, %d needed" % (st.idx.shape[1], k))
    bf16 = st.Kt.dtype == torch.bfloat16
    # anchors of this pass: the first k rows of the (contiguous) anchor buffers
    idx = st.idx.view(-1)[:G * k].view(G, k)
    Ka = st.K_anchor.view(-1)[:G * k * K.shape[2]].view(G, k, K.shape[2])
    Va = st.V_anchor.view(-1)[:G * k * K.shape[2]].view(G, k, K.shape[2])
    if reconstruct and fused:
        both = kvc.kvc_lowrank_compress_reconstruct_bf16 if bf16 else kvc.kvc_lowrank_compress_reconstruct
        place = kvc.kvc_place_anchors_bf16 if bf16 else kvc.kvc_place_anchors
        both(K, V, Q_win, U_k, U_v, L, B, H_kv, S=S, K_tilde=st.Kt, V_tilde=st.Vt, err=st.err,
             K_hat=st.Khat, V_hat=st.Vhat)
        kvc.kvc_topk_compact(st.err, k, K, V, S=S, idx_out=idx, K_out=Ka, V_out=Va)
        place(idx, Ka, L, B, H_kv, st.Khat, S=S)
        place(idx, Va, L, B, H_kv, st.Vhat, S=S)
        return idx, Ka, Va
    compress = kvc.kvc_lowrank_compress_bf16 if bf16 else kvc.kvc_lowrank_compress
    rebuild = kvc.kvc_reconstruct_bf16 if bf16 else kvc.kvc_reconstruct
    compress(K, V, Q_win, U_k, U_v, L, B, H_kv, S=S, K_tilde=st.Kt, V_tilde=st.Vt, err=st.err)
    kvc.kvc_topk_compact(st.err, k, K, V, S=S, idx_out=idx, K_out=Ka, V_out=Va)
    if reconstruct:
        rebuild(st.Kt, U_k, idx, Ka, L, B, H_kv, S=S, X_hat=st.Khat)
        rebuild(st.Vt, U_v, idx, Va, L, B, H_kv, S=S, X_hat=st.Vhat)
    return idx, Ka, Va


@dataclass
class OjaLoopState:
    U_k: torch.Tensor
    U_v: torch.Tensor
    hybrid: HybridState
    K_buf: torch.Tensor      # [G, T, D] tokens since the last update
    V_buf: torch.Tensor
    Q_dec: torch.Tensor      # [L, B, H_q, T, D] decode queries since the last update
    S: int                   # tokens in the cache
    step: int = 0
    updates: int = 0


def ojakv_prefill(K, V, Q_prompt, U_k, U_v, L, B, H_kv, S0, T=32, pool=32, eta=1e-3,
                  anchor_percent=5, S_cap=None, reconstruct=True, storage="fp32"):
    """Prefill phase (appendix A.1): pooled Oja update of U_k (on K) and U_v (on V)
    with QR, then projection, error score with the prompt's query window,
    top-k anchors and (optionally) reconstruction.  U_k, U_v are updated in place.
    K, V: bf16 [L*B*H_kv, S_cap, 128] caches holding S0 prompt tokens."""
    G, cap, D = K.shape
    S_cap = cap if S_cap is None else S_cap
    kvc.kvc_oja_update(U_k, K, pool, eta, L, B, H_kv, N=S0)
    kvc.kvc_oja_update(U_v, V, pool, eta, L, B, H_kv, N=S0)
    R = U_k.shape[-1]
    st = alloc_hybrid(G, S_cap, R, D, K.device, max_anchor=anchor_count(S_cap, anchor_percent),
                      with_hat=reconstruct, storage=storage)
    hybrid_pass(K, V, Q_prompt, U_k, U_v, L, B, H_kv, S0, st, anchor_percent, reconstruct)
    H_q = Q_prompt.shape[2]
    return OjaLoopState(
        U_k=U_k, U_v=U_v, hybrid=st,
        K_buf=torch.empty((G, T, D), dtype=torch.bfloat16, device=K.device),
        V_buf=torch.empty((G, T, D), dtype=torch.bfloat16, device=K.device),
        Q_dec=torch.empty((L, B, H_q, T, D), dtype=torch.bfloat16, device=K.device),
        S=S0)


def ojakv_decode_step(state: OjaLoopState, K, V, k_new, v_new, q_new, L, B, H_kv, T=32,
                      eta=1e-3, anchor_percent=5, reconstruct=True):
    """One decode step (appendix A.1): the new (k, v) are appended to the cache
    and to the update buffer, the new queries to the decode query window; when
    T tokens are buffered the bases take an unpooled Oja step + QR, and the
    whole cache is re-projected, re-scored with the T decode queries, its
    anchors re-selected and K^, V^ rebuilt.  Returns True on an update step.
    k_new, v_new: bf16 [G, 128]; q_new: bf16 [L, B, H_q, 128]."""
    slot = state.step % T
    kvc.kvc_decode_append(K, V, k_new, v_new, state.S, L, B, H_kv, K_buf=state.K_buf, V_buf=state.V_buf,
                          slot=slot, q_new=q_new, Q_buf=state.Q_dec)
    state.S += 1
    state.step += 1
    if state.step % T:
        return False
    kvc.kvc_oja_update(state.U_k, state.K_buf, 1, eta, L, B, H_kv)
    kvc.kvc_oja_update(state.U_v, state.V_buf, 1, eta, L, B, H_kv)
    hybrid_pass(K, V, state.Q_dec, state.U_k, state.U_v, L, B, H_kv, state.S, state.hybrid,
                anchor_percent, reconstruct)
    state.updates += 1
    return True
