"""Pins for the oracle's Oja basis update, pooling and QR.  Source: "OjaKV:
Context-Aware Online Low-Rank KV Cache Compression" deep-notes page -- the
Oja rule U <- U + eta (x x^T U - U U^T x x^T U) (how it works; method details),
pooled prefill update with the empirical covariance, re-orthonormalisation by
QR, appendix A.1's column-convention form of the same step."""
import numpy as np
import pytest

import oracle
import synth
from tests.helpers import bf16_bits_rne, int_bf16


def _basis(D, R, seed):
    # orthonormal to double precision (the fp32 bases of the workloads are not)
    Q, Rm = np.linalg.qr(np.random.default_rng(seed).standard_normal((D, R)))
    return Q * np.sign(np.diag(Rm))[None]


def test_step_equals_algorithm1_column_form():
    # Algorithm 1 writes, for feature columns K (d x n) and K~ = U^T K,
    # U + eta' (K - U K~) K~^T; with eta' = eta/n this is the covariance form.
    rng = np.random.default_rng(1)
    for n, D, R in [(7, 6, 2), (50, 16, 5), (3, 8, 8)]:
        X = rng.standard_normal((n, D))
        U = _basis(D, R, n)
        eta = 0.037
        Kc = X.T
        Kt = U.T @ Kc
        expect = U + (eta / n) * (Kc - U @ Kt) @ Kt.T
        np.testing.assert_allclose(oracle.oja_step(X, U, eta), expect, rtol=1e-12, atol=1e-13)


def test_eta_zero_and_fixed_point():
    rng = np.random.default_rng(2)
    D, R = 12, 4
    U = _basis(D, R, 5)
    X = rng.standard_normal((30, D))
    np.testing.assert_array_equal(oracle.oja_step(X, U, 0.0), U)
    # rows inside span(U): C U - U U^T C U = 0, the basis does not move
    Xin = rng.standard_normal((30, R)) @ U.T
    np.testing.assert_allclose(oracle.oja_step(Xin, U, 0.3), U, atol=1e-13)
    # and QR of an orthonormal basis with positive diagonal is itself
    np.testing.assert_allclose(oracle.qr(U), U, atol=1e-14)


def test_ascent_of_captured_variance():
    rng = np.random.default_rng(3)
    D, R = 10, 3
    X = rng.standard_normal((200, D)) * np.linspace(3, 0.2, D)
    C = X.T @ X / len(X)
    U = _basis(D, R, 6)
    for _ in range(20):
        Un = oracle.qr(oracle.oja_step(X, U, 0.01))
        assert np.trace(Un.T @ C @ Un) >= np.trace(U.T @ C @ U) - 1e-12
        U = Un


def test_converges_to_top_eigenspace():
    # repeated steps on a fixed covariance reach its top-r eigenspace (numpy.linalg.eigh)
    rng = np.random.default_rng(4)
    D, R = 16, 4
    X = rng.standard_normal((400, D)) @ np.diag(np.r_[np.full(R, 4.0), np.full(D - R, 1.0)]) @ \
        np.linalg.qr(rng.standard_normal((D, D)))[0]
    C = X.T @ X / len(X)
    w, Vecs = np.linalg.eigh(C)
    top = Vecs[:, np.argsort(w)[::-1][:R]]
    U = _basis(D, R, 7)
    for _ in range(400):
        U = oracle.qr(oracle.oja_step(X, U, 0.02))
    overlap = np.linalg.norm(top.T @ U) ** 2 / R
    assert overlap > 1 - 1e-8


def test_qr_against_library():
    rng = np.random.default_rng(5)
    for D, R in [(4, 1), (8, 8), (128, 64), (30, 7)]:
        A = rng.standard_normal((D, R))
        Q = oracle.qr(A)
        Ql, Rl = np.linalg.qr(A)
        Ql = Ql * np.sign(np.diag(Rl))[None]
        np.testing.assert_allclose(Q, Ql, atol=1e-12)
        np.testing.assert_allclose(Q.T @ Q, np.eye(R), atol=1e-13)
        Rm = Q.T @ A
        assert np.all(np.abs(np.tril(Rm, -1)) < 1e-11) and np.all(np.diag(Rm) > 0)
    with pytest.raises(ValueError):
        oracle.qr(np.zeros((4, 2)))


def test_pooling_closed_forms():
    rng = np.random.default_rng(6)
    X = int_bf16(rng.integers(-100, 101, size=(10, 3)))
    Xf = oracle.bf16_to_f64(X)
    np.testing.assert_array_equal(oracle.avgpool(X, 1), Xf)
    np.testing.assert_allclose(oracle.avgpool(X, 10), Xf.mean(0, keepdims=True), rtol=1e-15)
    # p=4 over 10 rows: windows [0,4) [4,8) and the short tail [8,10)
    P = oracle.avgpool(X, 4)
    np.testing.assert_allclose(P, np.stack([Xf[0:4].mean(0), Xf[4:8].mean(0), Xf[8:10].mean(0)]), rtol=1e-15)


def test_update_is_pool_step_qr_per_head():
    # oja_update = QR(step(pooled rows of every sequence of the batch, stacked)), per (layer, kv head)
    L, B, Hkv, N, D, R, p = 2, 3, 2, 37, 8, 3, 4
    rng = np.random.default_rng(7)
    X = bf16_bits_rne(rng.standard_normal((L * B * Hkv, N, D)) * 2)
    U = np.stack([np.stack([synth.orthonormal_basis(D, R, 9, l, h) for h in range(Hkv)]) for l in range(L)])
    eta = 0.05
    out = oracle.oja_update(U, X, p, eta, L, B, Hkv)
    Xf = oracle.bf16_to_f64(X)
    for l in range(L):
        for h in range(Hkv):
            rows = []
            for b in range(B):
                xs = Xf[(l * B + b) * Hkv + h]
                rows += [xs[i:i + p].mean(0) for i in range(0, N, p)]
            Xp = np.array(rows)
            C = Xp.T @ Xp / len(Xp)
            U0 = U[l, h].astype(np.float64)
            Un = U0 + eta * (C @ U0 - U0 @ (U0.T @ C @ U0))
            Ql, Rl = np.linalg.qr(Un)
            Ql = Ql * np.sign(np.diag(Rl))[None]
            np.testing.assert_allclose(out[l, h], Ql, atol=1e-12)


def test_full_loop_structure_small():
    # prefill + 2 decode updates on one slice: bases stay orthonormal, anchors are
    # ceil(5%) of the current length, reconstructed anchors equal their keys
    D, R, g, Wq, S0, steps, T = 16, 4, 2, 4, 64, 8, 4
    rng = np.random.default_rng(8)
    K = bf16_bits_rne(rng.standard_normal((S0 + steps, D)) + 1)
    V = bf16_bits_rne(rng.standard_normal((S0 + steps, D)) - 1)
    Qp = bf16_bits_rne(rng.standard_normal((g, Wq, D)))
    Qd = bf16_bits_rne(rng.standard_normal((steps, g, D)))
    Uk = synth.orthonormal_basis(D, R, 1)
    Uv = synth.orthonormal_basis(D, R, 2)
    res = oracle.full_loop_slice(K, V, Qp, Qd, Uk, Uv, S0, steps, T, pool=4, eta=1e-3)
    assert [r["S"] for r in res] == [64, 68, 72]
    for r in res:
        np.testing.assert_allclose(r["Uk"].astype(np.float64).T @ r["Uk"], np.eye(R), atol=1e-6)
        assert r["idx"].shape == (1, oracle.n_anchors(r["S"]))
        np.testing.assert_array_equal(r["Khat"][0][r["idx"][0]], oracle.bf16_to_f64(K[r["idx"][0]]))
