"""Pins for the oracle's RefineKV cluster summaries and risk score ("RefineKV"
project page: "Summarize" -- contiguous clusters with mean keys, mean values and
metadata -- and the Figure 2 formula RC = 2 p Vmax [(cosh d - 1)/Dn + tanh(d/2)]).
Summaries are pinned against numpy (means, norms); the risk score against closed
forms.  The page leaves p (share of attention mass) and d (logit-deviation bound)
without formulas: their readings are the oracle's, so RC is parity unpinned
relative to the pages beyond these closed forms (in particular RC is not checked
to bound the single-cluster replacement error)."""
import numpy as np
import pytest
from scipy.special import softmax

import oracle
from tests.helpers import int_bf16


def _kv(G, S, D, seed):
    rng = np.random.default_rng(seed)
    return int_bf16(rng.integers(-40, 41, size=(G, S, D))), int_bf16(rng.integers(-40, 41, size=(G, S, D)))


def test_summaries_match_numpy():
    for S, c in [(105, 10), (64, 64), (7, 100), (50, 1), (257, 32)]:
        K, V = _kv(2, S, 16, S + c)
        mk, mv, rad, vn = oracle.cluster_summaries(K, V, c)
        Kf, Vf = oracle.bf16_to_f64(K), oracle.bf16_to_f64(V)
        nC = -(-S // c)
        assert mk.shape == (2, nC, 16) and rad.shape == (2, nC)
        for g in range(2):
            for j in range(nC):
                kc, vc = Kf[g, j * c:(j + 1) * c], Vf[g, j * c:(j + 1) * c]
                np.testing.assert_allclose(mk[g, j], kc.mean(axis=0), rtol=1e-13, atol=1e-13)
                np.testing.assert_allclose(mv[g, j], vc.mean(axis=0), rtol=1e-13, atol=1e-13)
                assert rad[g, j] == pytest.approx(np.linalg.norm(kc - kc.mean(axis=0), axis=1).max(), rel=1e-12, abs=1e-12)
                assert vn[g, j] == pytest.approx(np.linalg.norm(vc, axis=1).max(), rel=1e-12)
        if c == 1:
            assert np.all(rad == 0.0)


def _q(G, nq, D, seed, scale=1.0):
    rng = np.random.default_rng(seed)
    x = np.round(rng.normal(0.0, scale, (G, nq, D)) * 16) / 16
    return int_bf16(x)


def test_single_cluster_closed_form():
    # one cluster: p = 1, Dn = cosh d  ->  RC = 2 Vmax [(cosh d - 1)/cosh d + tanh(d/2)]
    K, V = _kv(1, 40, 16, 3)
    mk, _, rad, vn = oracle.cluster_summaries(K, V, 40)
    Q = _q(1, 3, 16, 4, 0.3)
    rc = oracle.refine_risk(mk, rad, vn, 40, 40, Q)
    qf = oracle.bf16_to_f64(Q)[0]
    for i in range(3):
        d = np.linalg.norm(qf[i]) * rad[0, 0] / 4.0
        ref = 2.0 * vn[0, 0] * ((np.cosh(d) - 1.0) / np.cosh(d) + np.tanh(d / 2.0))
        assert rc[0, i, 0] == pytest.approx(ref, rel=1e-12)


def test_zero_deviation_or_zero_query_gives_zero_risk():
    K, V = _kv(2, 100, 16, 5)
    mk, _, rad, vn = oracle.cluster_summaries(K, V, 10)
    Q = _q(2, 2, 16, 6)
    assert np.all(oracle.refine_risk(mk, np.zeros_like(rad), vn, 100, 10, Q) == 0.0)
    assert np.all(oracle.refine_risk(mk, rad, vn, 100, 10, np.zeros_like(Q)) == 0.0)


def test_equal_radii_share_the_mass_by_softmax():
    # equal radii -> equal d: Dn = cosh d, RC_C = 2 p_C Vmax [...] with p the size-weighted
    # softmax of the representatives' logits (scipy), and sum_C RC_C = 2 Vmax [...]
    S, c, D = 95, 10, 16
    K, V = _kv(1, S, D, 7)
    mk, _, rad, vn = oracle.cluster_summaries(K, V, c)
    r0 = np.full_like(rad, 1.5)
    Q = _q(1, 2, D, 8, 0.2)
    rc = oracle.refine_risk(mk, r0, vn, S, c, Q)
    qf = oracle.bf16_to_f64(Q)[0]
    n = np.array([min(c, S - j * c) for j in range(mk.shape[1])], np.float64)
    vmax = vn.max()
    for i in range(2):
        d = np.linalg.norm(qf[i]) * 1.5 / np.sqrt(D)
        p = softmax(mk[0] @ qf[i] / np.sqrt(D) + np.log(n))
        scale = 2.0 * vmax * ((np.cosh(d) - 1.0) / np.cosh(d) + np.tanh(d / 2.0))
        np.testing.assert_allclose(rc[0, i], p * scale, rtol=1e-11)
        assert rc[0, i].sum() == pytest.approx(scale, rel=1e-12)
