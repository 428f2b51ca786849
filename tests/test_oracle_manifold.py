"""Pins for the oracle's ManifoldKV scorer (global and windowed), independent of
the oracle's own code: exact-rational brute force, closed forms, invariances
and a library identity.  Source: "ManifoldKV: Training-Free KV Cache
Compression via Euclidean Outlier Detection", abstract (Euclidean distance of
each key to the key centroid; WindowedManifoldKV's per-window centroid)."""
from fractions import Fraction

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import oracle
from tests.helpers import f64_to_bf16_bits_exact, int_bf16


def test_exact_rational_bruteforce_tiny():
    # integer-valued keys are exact in bf16; mean and squared distances are exact rationals
    rng = np.random.default_rng(1)
    for S, D in [(1, 1), (2, 3), (5, 4), (17, 8)]:
        Kint = rng.integers(-40, 41, size=(2, S, D))
        s, mu = oracle.score_l2(int_bf16(Kint))
        for g in range(2):
            mu_exact = [Fraction(int(Kint[g, :, c].sum()), S) for c in range(D)]
            for c in range(D):
                assert mu[g, c] == float(mu_exact[c]) or abs(mu[g, c] - float(mu_exact[c])) <= 1e-15 * max(1, abs(float(mu_exact[c])))
            for t in range(S):
                sq = sum((Fraction(int(Kint[g, t, c])) - mu_exact[c]) ** 2 for c in range(D))
                assert s[g, t] == pytest.approx(float(sq) ** 0.5, rel=1e-14, abs=1e-300)


def test_closed_form_line_through_centroid():
    # keys k_t = m + a_t e_1  ->  centroid m + mean(a) e_1,  s_t = |a_t - mean(a)|
    a = np.array([-3.0, 1.0, 2.0, 8.0, 0.0, -0.5, 4.0, 0.5])
    m = np.array([2.0, -1.0, 0.25, 6.0])
    K = np.tile(m, (len(a), 1))
    K[:, 0] += a
    s, mu = oracle.score_l2(f64_to_bf16_bits_exact(K)[None])
    np.testing.assert_allclose(s[0], np.abs(a - a.mean()), rtol=1e-15, atol=1e-15)
    np.testing.assert_allclose(mu[0], m + np.array([a.mean(), 0, 0, 0]), rtol=1e-15)


def test_mean_square_score_is_total_variance():
    # mean_t ||k_t - mu||^2 equals the sum of per-channel population variances (numpy.var)
    rng = np.random.default_rng(2)
    K = int_bf16(rng.integers(-100, 101, size=(3, 257, 16)))
    s, _ = oracle.score_l2(K)
    Kf = oracle.bf16_to_f64(K)
    np.testing.assert_allclose((s ** 2).mean(axis=1), Kf.var(axis=1).sum(axis=1), rtol=1e-12)


@settings(max_examples=25, deadline=None)
@given(S=st.integers(1, 40), D=st.integers(1, 12), seed=st.integers(0, 10**6),
       shift=st.integers(-16, 16), scale_exp=st.integers(-3, 3))
def test_translation_scaling_permutation(S, D, seed, shift, scale_exp):
    rng = np.random.default_rng(seed)
    Kint = rng.integers(-64, 65, size=(1, S, D))
    s0, _ = oracle.score_l2(int_bf16(Kint))
    # translation by an integer vector stays exact in bf16 (|values| <= 128 < 256)
    c = rng.integers(-abs(shift), abs(shift) + 1, size=D)
    s1, _ = oracle.score_l2(int_bf16(Kint + c))
    np.testing.assert_allclose(s1, s0, rtol=1e-13, atol=1e-12)
    # scaling by a power of two is exact; distances scale by |alpha|
    alpha = 2.0 ** scale_exp
    s2, _ = oracle.score_l2(f64_to_bf16_bits_exact(Kint * -alpha))
    np.testing.assert_allclose(s2, s0 * alpha, rtol=1e-13, atol=1e-12)
    # permuting tokens permutes the scores (the global centroid is order-free)
    perm = rng.permutation(S)
    s3, _ = oracle.score_l2(int_bf16(Kint[:, perm]))
    np.testing.assert_allclose(s3[0], s0[0, perm], rtol=1e-13, atol=1e-12)


def test_windowed_equals_global_when_window_covers_slice():
    rng = np.random.default_rng(3)
    K = int_bf16(rng.integers(-50, 51, size=(2, 37, 8)))
    sg, mug = oracle.score_l2(K)
    for W in (37, 38, 1000):
        sw, muw = oracle.score_l2_windowed(K, W)
        np.testing.assert_array_equal(sw, sg)
        np.testing.assert_array_equal(muw[:, 0], mug)


def test_windowed_w1_is_zero_and_windows_are_independent():
    rng = np.random.default_rng(4)
    K = int_bf16(rng.integers(-50, 51, size=(2, 30, 8)))
    sw, _ = oracle.score_l2_windowed(K, 1)
    assert np.all(sw == 0.0)
    # each window scores exactly like the global scorer applied to that window alone,
    # including the short tail window (30 = 3*8 + 6)
    W = 8
    sw, muw = oracle.score_l2_windowed(K, W)
    assert muw.shape == (2, 4, 8)
    for j in range(4):
        part = K[:, j * W:(j + 1) * W]
        sg, mug = oracle.score_l2(part)
        np.testing.assert_array_equal(sw[:, j * W:j * W + part.shape[1]], sg)
        np.testing.assert_array_equal(muw[:, j], mug)


def test_planted_outliers_rank_high():
    # generator sanity on a small config-0-like slice: the x4 tokens sit far from the centroid
    import synth
    K, _, plant = synth.manifold_global(1, 1, 2, 1024, planted=8)
    s, _ = oracle.score_l2(synth.bf16_bits(K))
    for g in range(2):
        order = np.argsort(-s[g], kind="stable")
        assert set(plant[g].tolist()) <= set(order[:int(0.8 * 1024)].tolist())
        assert np.median(s[g, plant[g].numpy()]) > 1.5 * np.median(s[g])


def test_nonfinite_rejected():
    K = int_bf16(np.ones((1, 4, 4), dtype=np.int64))
    K[0, 2, 1] = 0x7FC0  # NaN
    with pytest.raises(ValueError):
        oracle.score_l2(K)
    with pytest.raises(ValueError):
        oracle.score_l2_windowed(K, 2)
