"""Pins for the oracle's hybrid low-rank path: projection, residual, error score
and reconstruction.  Source: "OjaKV: Context-Aware Online Low-Rank KV Cache
Compression" deep-notes page -- background (K~ = K U_k, K^ = K~ U_k^T),
method details (r_t = k_t - U_k U_k^T k_t, the query-weighted error score e_t,
Cauchy-Schwarz bound), appendix A.4 (logit equivalence, memory saving
1 - (r_k + r_v)/(2 d_h)) and A.9 (commutation with token selection)."""
import numpy as np
import pytest

import oracle
import synth
from tests.helpers import f64_to_bf16_bits_exact, int_bf16


def _small(L=1, B=2, Hkv=2, Hq=8, S=40, D=16, R=8, Wq=4, seed=11):
    inp = synth.oja_inputs(L, B, Hkv, Hq, S, D=D, R=R, Wq=Wq, seed=seed)
    return (synth.bf16_bits(inp.K), synth.bf16_bits(inp.V), synth.bf16_bits(inp.Q),
            inp.Uk.numpy(), inp.Uv.numpy(), inp)


def test_identity_prefix_basis_closed_form():
    # U = first r standard basis vectors: k~ = k[:r], r_t = (0, k[r:]),
    # e_t = mean over the group's window of |q[r:] . k[r:]| / sqrt(d)
    K, V, Q, _, _, inp = _small()
    L, B, Hkv, Hq, S, D, R, Wq = inp.L, inp.B, inp.Hkv, inp.Hq, inp.S, inp.D, inp.R, inp.Wq
    E = np.zeros((L, Hkv, D, R), np.float32)
    E[..., np.arange(R), np.arange(R)] = 1.0
    Kt, Vt, err = oracle.lowrank_compress(K, V, Q, E, E, L, B, Hkv, Hq)
    Kf = oracle.bf16_to_f64(K)
    Qf = oracle.bf16_to_f64(Q)
    np.testing.assert_array_equal(Kt, Kf[..., :R])
    np.testing.assert_array_equal(Vt, oracle.bf16_to_f64(V)[..., :R])
    g = Hq // Hkv
    for l in range(L):
        for b in range(B):
            for h in range(Hkv):
                sl = (l * B + b) * Hkv + h
                q = Qf[l, b, h * g:(h + 1) * g].reshape(g * Wq, D)[:, R:]
                expect = np.abs(Kf[sl][:, R:] @ q.T).mean(axis=1) / np.sqrt(D)
                np.testing.assert_allclose(err[sl], expect, rtol=1e-13)


def test_projector_form_general_basis():
    # e_t = mean |q^T (I - U U^T) k_t| / sqrt(d): the same quantity through the
    # projector and library matmuls (valid for any U, orthonormal or not)
    K, V, Q, Uk, Uv, inp = _small(seed=12)
    L, B, Hkv, Hq, D, Wq = inp.L, inp.B, inp.Hkv, inp.Hq, inp.D, inp.Wq
    Uk = Uk + np.float32(0.01)  # break orthonormality on purpose
    Kt, Vt, err = oracle.lowrank_compress(K, V, Q, Uk, Uv, L, B, Hkv, Hq)
    Kf, Vf, Qf = (oracle.bf16_to_f64(x) for x in (K, V, Q))
    g = Hq // Hkv
    for b in range(B):
        for h in range(Hkv):
            sl = b * Hkv + h
            U = Uk[0, h].astype(np.float64)
            P = np.eye(D) - U @ U.T
            q = Qf[0, b, h * g:(h + 1) * g].reshape(g * Wq, D)
            np.testing.assert_allclose(err[sl], np.abs(Kf[sl] @ P @ q.T).mean(1) / np.sqrt(D), rtol=1e-11)
            np.testing.assert_allclose(Kt[sl], Kf[sl] @ U, rtol=1e-12, atol=1e-12)
            np.testing.assert_allclose(Vt[sl], Vf[sl] @ Uv[0, h].astype(np.float64), rtol=1e-12, atol=1e-12)


def test_keys_in_span_have_zero_residual():
    # Hadamard columns / 2 are an exactly representable orthonormal basis of R^4
    H = 0.5 * np.array([[1, 1, 1, 1], [1, -1, 1, -1], [1, 1, -1, -1], [1, -1, -1, 1]], np.float64)
    U = H[:, :2].astype(np.float32)[None, None]
    coeffs = np.array([[2, 4], [-6, 8], [0, 2], [10, -2], [1, 1]], np.float64)
    Kspan = coeffs @ H[:, :2].T
    K = f64_to_bf16_bits_exact(Kspan)[None]
    Q = int_bf16(np.arange(1, 1 + 2 * 3 * 4).reshape(1, 1, 2, 3, 4) % 7 - 3)
    Kt, _, err = oracle.lowrank_compress(K, None, Q, U, None, 1, 1, 1, 2)
    np.testing.assert_array_equal(err, 0.0)
    np.testing.assert_allclose(Kt[0], coeffs, rtol=0, atol=1e-15)
    # and they reconstruct to themselves
    Kh = oracle.reconstruct(Kt, U, None, None, 1, 1, 1)
    np.testing.assert_allclose(Kh[0], Kspan, atol=1e-14)
    # full rank basis (r = d): no residual for any key
    Kr = int_bf16(np.random.default_rng(0).integers(-9, 10, size=(1, 6, 4)))
    _, _, err = oracle.lowrank_compress(Kr, None, Q, H.astype(np.float32)[None, None], None, 1, 1, 1, 2)
    assert np.max(np.abs(err)) < 1e-14


def test_cauchy_schwarz_bound():
    # |q . r_t| / sqrt(d) <= ||q|| ||r_t|| / sqrt(d) term by term, hence for the mean
    K, V, Q, Uk, Uv, inp = _small(seed=13, S=64)
    Kt, _, err = oracle.lowrank_compress(K, None, Q, Uk, None, inp.L, inp.B, inp.Hkv, inp.Hq)
    Kh = oracle.reconstruct(Kt, Uk, None, None, inp.L, inp.B, inp.Hkv)
    r = oracle.bf16_to_f64(K) - Kh
    Qf = oracle.bf16_to_f64(Q)
    g = inp.Hq // inp.Hkv
    for b in range(inp.B):
        for h in range(inp.Hkv):
            sl = b * inp.Hkv + h
            qn = np.linalg.norm(Qf[0, b, h * g:(h + 1) * g], axis=-1).mean()
            bound = qn * np.linalg.norm(r[sl], axis=1) / np.sqrt(inp.D)
            assert np.all(err[sl] <= bound * (1 + 1e-12))
            assert np.all(err[sl] > 0)


def test_gqa_group_mapping():
    # kv head h reads query heads [h*g, (h+1)*g): zeroing a group zeroes exactly its head
    K, V, Q, Uk, Uv, inp = _small(seed=14, B=1)
    g = inp.Hq // inp.Hkv
    for h in range(inp.Hkv):
        Qz = Q.copy()
        Qz[0, 0, h * g:(h + 1) * g] = 0
        _, _, err = oracle.lowrank_compress(K, None, Qz, Uk, None, 1, 1, inp.Hkv, inp.Hq)
        for h2 in range(inp.Hkv):
            assert np.all(err[h2] == 0.0) == (h2 == h)


def test_logit_equivalence_and_commutation():
    # Q K^T with K^ = K~ U^T equals (Q U) K~^T (A.4); compressing a token subset
    # equals taking that subset of the compressed cache (A.9)
    K, V, Q, Uk, Uv, inp = _small(seed=15, B=1)
    Kt, _, err = oracle.lowrank_compress(K, None, Q, Uk, None, 1, 1, inp.Hkv, inp.Hq)
    Kh = oracle.reconstruct(Kt, Uk, None, None, 1, 1, inp.Hkv)
    Qf = oracle.bf16_to_f64(Q)
    for h in range(inp.Hkv):
        U = Uk[0, h].astype(np.float64)
        q = Qf[0, 0, h * 4:(h + 1) * 4].reshape(-1, inp.D)
        np.testing.assert_allclose(q @ Kh[h].T, (q @ U) @ Kt[h].T, rtol=1e-11, atol=1e-11)
    sel = np.array([[3, 7, 8, 20, 39]] * inp.Hkv, np.int32)
    Ks = oracle.gather(K, sel)
    Kt2, _, err2 = oracle.lowrank_compress(Ks, None, Q, Uk, None, 1, 1, inp.Hkv, inp.Hq)
    np.testing.assert_array_equal(Kt2, np.take_along_axis(Kt, sel[..., None].astype(np.int64), 1))
    np.testing.assert_array_equal(err2, np.take_along_axis(err, sel.astype(np.int64), 1))


def test_reconstruct_library_form_and_anchor_rows():
    rng = np.random.default_rng(16)
    G, S, R, D = 4, 33, 8, 16
    Xt = synth.random_lowrank(G, S, R, seed=3).numpy()
    U = np.stack([synth.orthonormal_basis(D, R, 1, h) for h in range(2)])[None]  # L=1, Hkv=2
    idx = np.sort(np.stack([rng.choice(S, 5, replace=False) for _ in range(G)]), 1).astype(np.int32)
    rows = rng.integers(0, 0x7F00, size=(G, 5, D)).astype(np.uint16)
    Xh = oracle.reconstruct(Xt, U, idx, rows, 1, 2, 2)
    for g in range(G):
        h = g % 2
        ref = Xt[g].astype(np.float64) @ U[0, h].astype(np.float64).T
        anchor = np.zeros(S, bool)
        anchor[idx[g]] = True
        np.testing.assert_allclose(Xh[g][~anchor], ref[~anchor], rtol=1e-12, atol=1e-12)
        np.testing.assert_array_equal(Xh[g][idx[g]], oracle.bf16_to_f64(rows[g]))


def test_strided_slices_ignore_padding():
    K, V, Q, Uk, Uv, inp = _small(seed=17)
    pad = np.concatenate([K, np.full((K.shape[0], 5, K.shape[2]), 0x7FC0, np.uint16)], axis=1)
    a = oracle.lowrank_compress(K, V, Q, Uk, Uv, inp.L, inp.B, inp.Hkv, inp.Hq)
    vpad = np.concatenate([V, np.zeros((V.shape[0], 5, V.shape[2]), np.uint16)], axis=1)
    b = oracle.lowrank_compress(pad, vpad, Q, Uk, Uv, inp.L, inp.B, inp.Hkv, inp.Hq, S=inp.S)
    for x, y in zip(a, b):
        np.testing.assert_array_equal(x, y[:, :inp.S])


def test_memory_closed_forms():
    # A.4: saving 1 - (r_k + r_v)/(2 d_h) = 0.5 at r = 64, d_h = 128;
    # the full-rank cache of 32 layers x 8 kv heads x d_h 128 at 32K tokens x batch 4 in 16-bit is 16 GiB
    assert 1 - (64 + 64) / (2 * 128) == 0.5
    assert 2 * 32 * 8 * 128 * 2 * 32768 * 4 == 16 * 2 ** 30


def test_invalid_arguments():
    K, V, Q, Uk, Uv, inp = _small()
    with pytest.raises(ValueError):  # H_q not a multiple of H_kv
        oracle.lowrank_compress(K, V, Q, Uk, Uv, inp.L, inp.B, inp.Hkv, 7)
    with pytest.raises(ValueError):  # V without its basis
        oracle.lowrank_compress(K, V, Q, Uk, None, inp.L, inp.B, inp.Hkv, inp.Hq)


def _softmax(z):
    e = np.exp(z - z.max())
    return e / e.sum()


def test_attention_error_chain_on_hybrid_reconstruction():
    # appendix A.2's chain on the oracle's hybrid cache of one slice (anchors = the
    # top 5% of e_t, kept exact): for every query, |z^_t - z_t| <= ||q|| ||e_t|| / sqrt(d),
    # ||a^ - a||_1 <= 2 ||z^ - z||_inf, and ||o^ - o||_2 <= V ||a^ - a||_1 <= 2 V Q E / sqrt(d),
    # with exact values V; softmax attention in fp64.  A consistency check of the
    # reconstruction against the pages' bound (it holds for any residual); the
    # reconstruction itself is pinned by the library-form test above.
    K, V, Q, Uk, Uv, inp = _small(L=1, B=1, Hkv=1, Hq=4, S=300, D=128, R=16, Wq=8, seed=5)
    Kt, _, err = oracle.lowrank_compress(K, None, Q, Uk, None, 1, 1, 1, 4)
    k = oracle.n_anchors(300)
    idx = oracle.topk(err.astype(np.float32), k)
    Kh = oracle.reconstruct(Kt, Uk, idx, oracle.gather(K, idx), 1, 1, 1)[0]
    Kf = oracle.bf16_to_f64(K[0])
    Vf = oracle.bf16_to_f64(V[0])
    res = np.linalg.norm(Kh - Kf, axis=1)
    assert np.all(res[idx[0]] == 0.0)                       # anchors are exact
    E = res.max()
    Vb = np.linalg.norm(Vf, axis=1).max()
    d = 128
    rng = np.random.default_rng(9)
    for q in rng.normal(0.0, 1.0, (6, d)) * np.array([0.1, 1.0, 3.0, 10.0, 1.0, 0.5])[:, None]:
        z, zh = Kf @ q / np.sqrt(d), Kh @ q / np.sqrt(d)
        Qn = np.linalg.norm(q)
        assert np.all(np.abs(zh - z) <= Qn * res / np.sqrt(d) * (1 + 1e-12) + 1e-15)
        a, ah = _softmax(z), _softmax(zh)
        l1 = np.abs(ah - a).sum()
        assert l1 <= 2 * np.abs(zh - z).max() * (1 + 1e-9) + 1e-15
        do = np.linalg.norm(ah @ Vf - a @ Vf)
        assert do <= Vb * l1 * (1 + 1e-9) + 1e-15
        assert do <= 2 * Vb * Qn * E / np.sqrt(d) * (1 + 1e-9) + 1e-15
