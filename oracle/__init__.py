"""CPU oracle for KV-cache token scoring, compaction and hybrid low-rank compression.

TEST INFRASTRUCTURE ONLY: the test suite, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package; the product path
never does.  It shares no code with the HIP library: the arithmetic lives in
``kvc_oracle.c`` (plain single-threaded C, double precision), built with gcc;
this module only marshals numpy arrays.

Sources, by page title and section:
  * "ManifoldKV: Training-Free KV Cache Compression via Euclidean Outlier
    Detection", abstract: Euclidean distance of each key to the key centroid;
    the windowed variant scores against a per-window centroid; the farthest
    keys are retained.
  * "OjaKV: Context-Aware Online Low-Rank KV Cache Compression" (deep-notes
    page): low-rank projection and reconstruction (background), residual and
    query-weighted error score, top-k full-rank anchors, pooled prefill Oja
    update with QR, decode-time buffered updates (method details; appendix A.1).

Every function is pinned by the ``-m "not gpu"`` tests.  ``full_loop_slice`` is
pinned by a worked example of the whole loop (tests/golden/oja_loop_tiny.json:
pooled prefill update, QR, scoring with the updated bases, anchors, then two
decode updates with re-projection, re-scoring and re-selection, computed with
exact rationals and 60-digit decimals) that also tells apart planted mistakes
in the order of the steps, the pooling, the buffer and the query window.  What
stays a reading is its decode-time re-projection and re-selection over the
whole cache (the pages' decode phase re-projects nothing): that reading is
**parity unpinned relative to the pages**, though its arithmetic is pinned.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kvc_oracle.c")
# KVC_ORACLE_LIB names another build of the same source to load instead (the
# sanitizer test runs the pins against an AddressSanitizer/UBSan build this way)
_LIB = os.environ.get("KVC_ORACLE_LIB") or os.path.join(_HERE, "liboracle.so")
_lock = threading.Lock()
_lib = None

ORA_ERRORS = {-1: "invalid argument", -2: "non-finite input", -3: "out of memory"}


def build(force: bool = True) -> str:
    """Compile ``kvc_oracle.c`` into ``liboracle.so`` with gcc (-O2, no fast-math)."""
    if not force and os.path.exists(_LIB) and os.path.getmtime(_LIB) >= os.path.getmtime(_SRC):
        return _LIB
    tmp = _LIB + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-fno-fast-math", "-ffp-contract=off",
           "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    with _lock:
        if _lib is None:
            if not os.environ.get("KVC_ORACLE_LIB"):
                build(force=False)
            lib = ctypes.CDLL(_LIB)
            P = ctypes.c_void_p
            I = ctypes.c_int64
            D = ctypes.c_double
            sig = {
                "ora_score_l2": [P, I, I, I, P, P],
                "ora_score_l2_windowed": [P, I, I, I, I, P, P],
                "ora_score_cosine_windowed": [P, I, I, I, I, P, P],
                "ora_topk": [P, I, I, I, I, P],
                "ora_gather": [P, I, I, I, I, P, I, P],
                "ora_lowrank_compress": [I, I, I, I, I, I, I, I, I, P, P, P, P, P, P, P, P],
                "ora_reconstruct": [I, I, I, I, I, I, I, P, P, P, P, I, P],
                "ora_avgpool": [P, I, I, I, P],
                "ora_oja_step": [P, I, I, I, P, D, P],
                "ora_qr": [P, I, I, P],
                "ora_oja_update": [I, I, I, I, I, I, I, P, P, I, D, P],
                "ora_layer_budgets": [P, I, D, D, I, I, P],
                "ora_cluster_summaries": [P, P, I, I, I, I, P, P, P, P],
                "ora_refine_risk": [P, P, P, I, I, I, I, P, I, P],
            }
            for name, argtypes in sig.items():
                fn = getattr(lib, name)
                fn.argtypes = argtypes
                fn.restype = ctypes.c_int
            lib.ora_bf16_to_f64.argtypes = [ctypes.c_uint16]
            lib.ora_bf16_to_f64.restype = ctypes.c_double
            _lib = lib
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _check(rc, name):
    if rc != 0:
        raise ValueError("%s: %s" % (name, ORA_ERRORS.get(rc, "error %d" % rc)))


def _u16(a):
    a = np.ascontiguousarray(a)
    if a.dtype != np.uint16:
        raise TypeError("bf16 tensors are passed as their uint16 bit patterns")
    return a


def _f32(a):
    return np.ascontiguousarray(a, dtype=np.float32)


def _f64(a):
    return np.ascontiguousarray(a, dtype=np.float64)


# ----------------------------------------------------------------- ManifoldKV

def score_l2(K):
    """Global ManifoldKV score.  K: uint16 (bf16 bits) [G, S, D].
    Returns (scores float64 [G, S], centroid float64 [G, D])."""
    K = _u16(K)
    G, S, D = K.shape
    scores = np.zeros((G, S), np.float64)
    mu = np.zeros((G, D), np.float64)
    _check(_load().ora_score_l2(_p(K), G, S, D, _p(scores), _p(mu)), "score_l2")
    return scores, mu


def score_l2_windowed(K, W):
    """WindowedManifoldKV score with contiguous windows of W tokens.
    Returns (scores float64 [G, S], centroids float64 [G, ceil(S/W), D])."""
    K = _u16(K)
    G, S, D = K.shape
    nwin = -(-S // W) if W > 0 else 0
    scores = np.zeros((G, S), np.float64)
    mu = np.zeros((G, nwin, D), np.float64)
    _check(_load().ora_score_l2_windowed(_p(K), G, S, D, W, _p(scores), _p(mu)),
           "score_l2_windowed")
    return scores, mu


def score_cosine_windowed(K, W):
    """Cosine dissimilarity 1 - cos(k_t, mu) to the centroid of each contiguous
    window of W keys (W >= S: the global centroid).  Returns (scores float64
    [G, S], centroids float64 [G, ceil(S/W), D])."""
    K = _u16(K)
    G, S, D = K.shape
    nwin = -(-S // W) if W > 0 else 0
    scores = np.zeros((G, S), np.float64)
    mu = np.zeros((G, nwin, D), np.float64)
    _check(_load().ora_score_cosine_windowed(_p(K), G, S, D, W, _p(scores), _p(mu)),
           "score_cosine_windowed")
    return scores, mu


def score_cosine(K):
    """Cosine dissimilarity to the global key centroid.  Returns (scores float64
    [G, S], centroid float64 [G, D])."""
    K = _u16(K)
    G, S, D = K.shape
    scores, mu = score_cosine_windowed(K, max(S, 1))
    return scores, (mu[:, 0] if S > 0 else np.zeros((G, D), np.float64))


def topk(scores32, k, S=None):
    """Indices of the k largest fp32 scores per slice, ties to the lower index,
    returned ascending.  scores32: float32 [G, S_stride]; S defaults to S_stride."""
    s = _f32(scores32)
    G, stride = s.shape
    S = stride if S is None else S
    idx = np.zeros((G, k), np.int32)
    _check(_load().ora_topk(_p(s), G, S, stride, k, _p(idx)), "topk")
    return idx


def gather(X, idx, S=None):
    """Rows of X (uint16 [G, S_stride, D]) at idx (int32 [G, k]), bytes unchanged."""
    X = _u16(X)
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    G, stride, D = X.shape
    S = stride if S is None else S
    k = idx.shape[1]
    out = np.zeros((G, k, D), np.uint16)
    _check(_load().ora_gather(_p(X), G, S, stride, D, _p(idx), k, _p(out)), "gather")
    return out


def retained(scores32, k, K=None, V=None):
    """ManifoldKV eviction of one batch of slices: top-k then compaction."""
    idx = topk(scores32, k)
    return idx, (gather(K, idx) if K is not None else None), (gather(V, idx) if V is not None else None)


# ----------------------------------------------------------------------- OjaKV

def lowrank_compress(K, V, Q, Uk, Uv, L, B, Hkv, Hq, S=None):
    """Projection, residual and error score for every token.
    K, V: uint16 [L*B*Hkv, S_stride, D] (V may be None); Q: uint16
    [L, B, Hq, Wq, D] (None -> no score); Uk, Uv: float32 [L, Hkv, D, R].
    Returns (Kt [G,S_stride,R], Vt or None, err [G,S_stride] or None), float64."""
    K = _u16(K)
    G, stride, D = K.shape
    S = stride if S is None else S
    Uk = _f32(Uk)
    R = Uk.shape[-1]
    Wq = 0 if Q is None else Q.shape[-2]
    Q = None if Q is None else _u16(Q)
    V = None if V is None else _u16(V)
    Uv = None if Uv is None else _f32(Uv)
    Kt = np.zeros((G, stride, R), np.float64)
    Vt = None if V is None else np.zeros((G, stride, R), np.float64)
    err = None if Q is None else np.zeros((G, stride), np.float64)
    rc = _load().ora_lowrank_compress(L, B, Hkv, Hq, S, stride, D, R, Wq, _p(K), _p(V), _p(Q),
                                      _p(Uk), _p(Uv), _p(Kt), _p(Vt), _p(err))
    _check(rc, "lowrank_compress")
    return Kt, Vt, err


def reconstruct(Xt, U, idx, rows, L, B, Hkv, S=None):
    """X^ = X~ U^T, with anchor rows (bf16 bits) put back at their indices.
    Xt: [G, S_stride, R] (any float dtype, widened exactly); U: float32
    [L, Hkv, D, R]; idx: int32 [G, k] or None; rows: uint16 [G, k, D] or None."""
    Xt = _f64(Xt)
    G, stride, R = Xt.shape
    S = stride if S is None else S
    U = _f32(U)
    D = U.shape[-2]
    k = 0 if idx is None else idx.shape[1]
    idx = None if idx is None else np.ascontiguousarray(idx, dtype=np.int32)
    rows = None if rows is None else _u16(rows)
    out = np.zeros((G, stride, D), np.float64)
    rc = _load().ora_reconstruct(L, B, Hkv, S, stride, D, R, _p(Xt), _p(U), _p(idx), _p(rows),
                                 k, _p(out))
    _check(rc, "reconstruct")
    return out


def avgpool(X, p):
    """Average pooling of one slice's rows.  X: uint16 [N, D] -> float64 [ceil(N/p), D]."""
    X = _u16(X)
    N, D = X.shape
    out = np.zeros((-(-N // p), D), np.float64)
    _check(_load().ora_avgpool(_p(X), N, D, p, _p(out)), "avgpool")
    return out


def oja_step(X, U, eta):
    """One Oja step, no QR.  X: float64 [n, D] rows; U: float64 [D, R]."""
    X = _f64(X)
    U = _f64(U)
    n, D = X.shape
    R = U.shape[1]
    out = np.zeros((D, R), np.float64)
    _check(_load().ora_oja_step(_p(X), n, D, R, _p(U), float(eta), _p(out)), "oja_step")
    return out


def qr(A):
    """Thin QR factor Q (positive diagonal of R) of A: float64 [D, R]."""
    A = _f64(A)
    D, R = A.shape
    Q = np.zeros((D, R), np.float64)
    _check(_load().ora_qr(_p(A), D, R, _p(Q)), "qr")
    return Q


def oja_update(U, X, pool, eta, L, B, Hkv, N=None):
    """Pool -> Oja step -> QR for every (layer, kv head).
    U: float32 [L, Hkv, D, R]; X: uint16 [L*B*Hkv, N_stride, D].
    Returns the new basis in float64 [L, Hkv, D, R]."""
    U = _f32(U)
    X = _u16(X)
    _, stride, D = X.shape
    N = stride if N is None else N
    R = U.shape[-1]
    out = np.zeros(U.shape, np.float64)
    rc = _load().ora_oja_update(L, B, Hkv, N, stride, D, R, _p(U), _p(X), pool, float(eta), _p(out))
    _check(rc, "oja_update")
    return out


def n_anchors(S, percent=5):
    """Anchor count for a 'top p% of tokens' budget: ceil(p*S/100)."""
    return -(-percent * S // 100)


def keep_count(S, drop_percent):
    """Tokens kept when x% of S are evicted: S - floor(x*S/100) = ceil((100-x)*S/100)."""
    return S - (drop_percent * S) // 100


def hybrid_compress_slice(K, V, Q, Uk, Uv, k_anchor, S=None):
    """One (layer, batch, kv head) of the hybrid cache: compress, score, pick
    anchors on the fp32-rounded error score, reconstruct K^ and V^.
    Shapes: K, V [1, S, D]; Q [1, 1, g, Wq, D]; Uk, Uv [1, 1, D, R]."""
    g = Q.shape[2]
    Kt, Vt, err = lowrank_compress(K, V, Q, Uk, Uv, 1, 1, 1, g, S=S)
    idx = topk(err.astype(np.float32), k_anchor, S=S)
    Kh = reconstruct(Kt, Uk, idx, gather(K, idx, S=S), 1, 1, 1, S=S)
    Vh = reconstruct(Vt, Uv, idx, gather(V, idx, S=S), 1, 1, 1, S=S)
    return dict(Kt=Kt, Vt=Vt, err=err, idx=idx, Khat=Kh, Vhat=Vh)


def full_loop_slice(K, V, Qprompt, Qdec, Uk, Uv, S0, steps, T, pool, eta, anchor_percent=5,
                    on_update=None):
    """The prefill + decode loop of appendix A.1 on one (layer, kv head) with
    batch 1, following the pages' order: prefill pooled Oja update of U_k and
    U_v, QR, score with the updated basis, top-k anchors; then every T decode
    steps an update on the T buffered tokens (no pooling), QR, buffer reset.

    The re-projection, re-scoring and re-selection over the whole cache at each
    decode update (and the use of the T decode queries as the query window) is
    the reading adopted here for the full-loop workload: the pages' decode phase
    re-projects nothing.  Parity unpinned relative to the pages; the arithmetic
    and the order of the steps are pinned by the loop's worked example.

    K, V: uint16 [S0+steps, D] (the full-rank rows the caller keeps);
    Qprompt: uint16 [g, Wq, D]; Qdec: uint16 [steps, g, D];
    Uk, Uv: float32 [D, R].  The basis is stored in fp32 between updates.
    ``on_update(j, state)`` is called after the prefill (j=0) and each update."""
    D = K.shape[1]
    g = Qprompt.shape[0]
    Uk = np.asarray(Uk, np.float32).reshape(1, 1, D, -1)
    Uv = np.asarray(Uv, np.float32).reshape(1, 1, D, -1)
    Kp = K[None, :S0]
    Vp = V[None, :S0]
    Uk = oja_update(Uk, Kp, pool, eta, 1, 1, 1).astype(np.float32)
    Uv = oja_update(Uv, Vp, pool, eta, 1, 1, 1).astype(np.float32)
    st = hybrid_compress_slice(Kp, Vp, Qprompt[None, None], Uk, Uv, n_anchors(S0, anchor_percent))
    st.update(Uk=Uk[0, 0], Uv=Uv[0, 0], S=S0)
    results = [st]
    if on_update:
        on_update(0, st)
    for j in range(1, steps // T + 1):
        S = S0 + j * T
        buf_k = K[None, S - T:S]
        buf_v = V[None, S - T:S]
        Uk = oja_update(Uk, buf_k, 1, eta, 1, 1, 1).astype(np.float32)
        Uv = oja_update(Uv, buf_v, 1, eta, 1, 1, 1).astype(np.float32)
        qwin = np.ascontiguousarray(Qdec[S - T - S0:S - S0].transpose(1, 0, 2))  # [g, T, D]
        st = hybrid_compress_slice(K[None, :S], V[None, :S], qwin[None, None], Uk, Uv,
                                   n_anchors(S, anchor_percent))
        st.update(Uk=Uk[0, 0], Uv=Uv[0, 0], S=S)
        results.append(st)
        if on_update:
            on_update(j, st)
    return results


def bf16_to_f64(bits):
    """Exact widening of bf16 bit patterns (uint16) to float64."""
    b = np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def layer_budgets(sensitivity, r, gamma, B, S):
    """RippleKV per-layer budgets: normalised sensitivities, multipliers r^s
    clipped to [1/gamma, gamma], rescaled to sum to B (budgets above S capped and
    re-spread; integers by largest remainder).  Returns int64 [L]."""
    s = np.ascontiguousarray(sensitivity, dtype=np.float64)
    k = np.zeros(s.shape[0], np.int64)
    _check(_load().ora_layer_budgets(_p(s), s.shape[0], float(r), float(gamma), int(B), int(S), _p(k)),
           "layer_budgets")
    return k


def topk_ragged(scores32, ks, S=None):
    """Top-k per slice with a budget per slice (ks: int [G]); indices packed in
    slice order: slice g's ks[g] ascending indices, then slice g+1's."""
    s = _f32(scores32)
    parts = [topk(s[g:g + 1], int(ks[g]), S)[0] for g in range(s.shape[0])]
    return np.concatenate(parts).astype(np.int32) if parts else np.zeros(0, np.int32)


def cluster_summaries(K, V, c):
    """RefineKV summaries of contiguous c-token clusters: (mu_k [G, nC, D],
    mu_v [G, nC, D], radius [G, nC], vnorm [G, nC]) in float64."""
    K, V = _u16(K), _u16(V)
    G, S, D = K.shape
    nC = -(-S // c)
    mk, mv = np.zeros((G, nC, D)), np.zeros((G, nC, D))
    rad, vn = np.zeros((G, nC)), np.zeros((G, nC))
    _check(_load().ora_cluster_summaries(_p(K), _p(V), G, S, D, c, _p(mk), _p(mv), _p(rad), _p(vn)),
           "cluster_summaries")
    return mk, mv, rad, vn


def refine_risk(mu_k, radius, vnorm, S, c, Q):
    """RefineKV risk scores RC [G, nq, nC] (float64) of every cluster for each
    query; Q: bf16 bits [G, nq, D]."""
    mu_k = np.ascontiguousarray(mu_k, np.float64)
    radius = np.ascontiguousarray(radius, np.float64)
    vnorm = np.ascontiguousarray(vnorm, np.float64)
    Q = _u16(Q)
    G, nC, D = mu_k.shape
    nq = Q.shape[1]
    rc = np.zeros((G, nq, nC))
    _check(_load().ora_refine_risk(_p(mu_k), _p(radius), _p(vnorm), G, S, c, D, _p(Q), nq, _p(rc)),
           "refine_risk")
    return rc

