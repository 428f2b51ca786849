"""Pins for the oracle's RefineKV cluster summaries and risk score ("RefineKV"
project page: "Summarize" -- contiguous clusters with mean keys, mean values and
metadata -- and the Figure 2 formula RC = 2 p Vmax [(cosh d - 1)/Dn + tanh(d/2)]).
Summaries are pinned against numpy (means, norms); the risk score against closed
forms, and against what the page says the scores are: the cluster-wise terms of an
upper bound on the attention-output error.  The page leaves p (share of attention
mass) and d (logit-deviation bound) without formulas; under the oracle's readings
the sum of the clusters' RC bounds the error of attending with every cluster
replaced by its size-weighted representative (mean key, mean value), checked on
random and adversarial instances (not proven here).  RC is not checked to bound the
single-cluster replacement error, which the page only correlates with it."""
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


def _bf16_rne(a):
    u = np.ascontiguousarray(a, np.float32).view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def _representative_error(K, V, Q, mk, mv, S, c):
    """||o - o'|| per query: exact attention output against the output with every
    cluster replaced by its mean key and mean value, weighted by its size."""
    Kf, Vf, Qf = oracle.bf16_to_f64(K)[0], oracle.bf16_to_f64(V)[0], oracle.bf16_to_f64(Q)[0]
    D = Kf.shape[1]
    n = np.array([min(c, S - j * c) for j in range(mk.shape[1])], np.float64)
    out = []
    for q in Qf:
        o = softmax(Kf @ q / np.sqrt(D)) @ Vf
        o2 = softmax(mk[0] @ q / np.sqrt(D) + np.log(n)) @ mv[0]
        out.append(np.linalg.norm(o - o2))
    return np.array(out)


def test_risk_scores_sum_to_a_bound_of_the_representative_error():
    # the page derives RC from an upper bound on attention-output error and uses its
    # cluster-wise terms as risk scores: with every cluster replaced by its
    # representative, the error must not exceed sum_C RC_C.  Random caches, and
    # adversarial ones where the bound is nearly attained: two-point clusters, values
    # following the key deviations, a query along the deviations, and one cluster of
    # large values beside spread-out clusters of small values.  A reading that makes
    # RC too small fails here: d with an extra 1/sqrt(d) or halved, Vmax taken per
    # cluster or as the mean value norm (checked when this test was written)
    rng = np.random.default_rng(2026)
    worst = 0.0
    for trial in range(1500):
        D = 16
        nC = int(rng.integers(1, 6))
        c = int(rng.integers(2, 12))
        S = max(1, nC * c - int(rng.integers(0, c)))
        kind = trial % 5
        base = rng.normal(0.0, float(rng.choice([0.5, 2.0, 6.0])), (nC, D))
        big = int(rng.integers(0, nC))
        K = np.zeros((1, S, D))
        V = np.zeros((1, S, D))
        for t in range(S):
            C, sign = t // c, (1.0 if t % 2 == 0 else -1.0)
            if kind == 0:
                K[0, t] = base[C] + sign * rng.normal(0.0, 1.0, D) * float(rng.choice([0.5, 2.0, 5.0]))
            elif kind == 1:
                K[0, t] = base[C] + rng.normal(0.0, float(rng.choice([0.1, 1.0, 4.0])), D)
            elif kind == 4:
                K[0, t] = base[C] + (0.0 if C == big else sign * float(rng.choice([1.0, 3.0])))
            else:
                K[0, t] = base[C] + sign * float(rng.choice([0.3, 1.0, 3.0]))
            if kind == 4:
                V[0, t] = (20.0 if C == big else 0.05) * rng.normal(0.0, 1.0, D)
            else:
                V[0, t] = (K[0, t] - base[C]) if kind >= 2 else rng.normal(0.0, 1.0, D)
        Q = rng.normal(0.0, float(rng.choice([0.1, 0.5, 1.5])), (1, 2, D))
        if kind in (3, 4):
            Q[0, 0] = float(rng.choice([0.2, 1.0]))
        Kb, Vb, Qb = _bf16_rne(K), _bf16_rne(V), _bf16_rne(Q)
        mk, mv, rad, vn = oracle.cluster_summaries(Kb, Vb, c)
        bound = oracle.refine_risk(mk, rad, vn, S, c, Qb)[0].sum(axis=1)
        err = _representative_error(Kb, Vb, Qb, mk, mv, S, c)
        # a bound of 0 (no spread) leaves only rounding in the error
        tol = 1e-12 * vn.max()
        assert np.all(err <= bound * (1 + 1e-12) + tol), (trial, err, bound)
        ratio = np.where(bound > 1e-9 * vn.max(), err / np.maximum(bound, 1e-300), 0.0)
        worst = max(worst, float(ratio.max()))
    # the check is tight enough to see a risk score half as large (a dropped factor,
    # or d or Vmax read too small by that much)
    assert worst > 0.5
