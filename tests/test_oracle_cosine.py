"""Pins for the oracle's cosine-dissimilarity scorer, s_t = 1 - cos(k_t, mu), the
geometry-based baseline the ManifoldKV abstract contrasts with its L2 score
("ManifoldKV: Training-Free KV Cache Compression via Euclidean Outlier
Detection", abstract: keys scored by cosine similarity to a global centroid,
cosine being scale-invariant).  Independent of the oracle's own code: a library
routine (scipy's cosine distance), closed forms in two dimensions, invariances
and the degenerate cases."""
import math

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st
from scipy.spatial.distance import cosine as scipy_cosine

import oracle
from tests.helpers import f64_to_bf16_bits_exact, int_bf16


def test_matches_scipy_cosine_distance():
    rng = np.random.default_rng(11)
    for S, D in [(1, 3), (7, 5), (64, 16), (300, 128)]:
        K = int_bf16(rng.integers(-50, 51, size=(2, S, D)))
        Kf = oracle.bf16_to_f64(K)
        s, mu = oracle.score_cosine(K)
        for g in range(2):
            m = Kf[g].mean(axis=0)
            np.testing.assert_allclose(mu[g], m, rtol=1e-13, atol=1e-13)
            ref = np.array([scipy_cosine(Kf[g, t], m) if np.any(Kf[g, t]) else 1.0 for t in range(S)])
            np.testing.assert_allclose(s[g], ref, rtol=1e-12, atol=1e-14)


def test_closed_form_angles_in_a_plane():
    # keys r_t (cos th_t, sin th_t, 0, ...): the centroid has angle phi = atan2(mean y, mean x),
    # and s_t = 1 - cos(th_t - phi) whatever the radii
    th = np.array([0.0, 0.5, 1.0, 2.5, -0.75, 3.0])
    r = np.array([1.0, 2.0, 0.5, 4.0, 1.5, 0.25])
    K = np.zeros((len(th), 8))
    K[:, 0] = r * np.cos(th)
    K[:, 1] = r * np.sin(th)
    bits = f64_to_bf16_bits_exact(np.round(K * 64) / 64)[None]  # |K| <= 4 on a 1/64 grid: 8 bits
    Kq = oracle.bf16_to_f64(bits)[0]
    phi = math.atan2(Kq[:, 1].mean(), Kq[:, 0].mean())
    ang = np.arctan2(Kq[:, 1], Kq[:, 0])
    s, _ = oracle.score_cosine(bits)
    np.testing.assert_allclose(s[0], 1.0 - np.cos(ang - phi), rtol=1e-12, atol=1e-14)


def test_parallel_keys_score_zero_and_orthogonal_keys_score_one():
    # keys a, a, 3a, b, -b: the centroid is a; a and 3a are parallel to it (s = 0),
    # +-b are orthogonal (s = 1)
    a = np.array([1.0, 2.0, 0.0, -1.0])
    b = np.array([2.0, -1.0, 4.0, 0.0])  # a . b = 0
    K = np.stack([a, a, 3 * a, b, -b])
    s, mu = oracle.score_cosine(f64_to_bf16_bits_exact(K)[None])
    np.testing.assert_allclose(mu[0], a, rtol=1e-15)
    np.testing.assert_allclose(s[0], [0.0, 0.0, 0.0, 1.0, 1.0], atol=1e-15)


def test_zero_key_or_zero_centroid_scores_one():
    K = np.array([[1.0, 0.0], [-1.0, 0.0], [0.0, 0.0]])  # centroid exactly zero
    s, _ = oracle.score_cosine(f64_to_bf16_bits_exact(K)[None])
    assert np.all(s[0] == 1.0)
    K = np.array([[1.0, 1.0], [0.0, 0.0], [3.0, 1.0]])  # a zero key, nonzero centroid
    s, _ = oracle.score_cosine(f64_to_bf16_bits_exact(K)[None])
    assert s[0, 1] == 1.0 and s[0, 0] < 1.0


@settings(max_examples=25, deadline=None)
@given(S=st.integers(1, 40), D=st.integers(2, 12), seed=st.integers(0, 10**6), e=st.integers(-6, 6))
def test_scale_invariance(S, D, seed, e):
    # cosine ignores magnitude: scaling every key by 2^e (exact in bf16) changes nothing;
    # the L2 score scales by 2^e
    rng = np.random.default_rng(seed)
    Kint = rng.integers(-64, 65, size=(1, S, D))
    s0, _ = oracle.score_cosine(int_bf16(Kint))
    s1, _ = oracle.score_cosine(f64_to_bf16_bits_exact(Kint * 2.0 ** e))
    np.testing.assert_allclose(s1, s0, rtol=1e-12, atol=1e-15)
    l0, _ = oracle.score_l2(int_bf16(Kint))
    l1, _ = oracle.score_l2(f64_to_bf16_bits_exact(Kint * 2.0 ** e))
    np.testing.assert_allclose(l1, l0 * 2.0 ** e, rtol=1e-12, atol=1e-300)


def test_windowed_reduces_to_global_and_to_each_window():
    rng = np.random.default_rng(5)
    K = int_bf16(rng.integers(-30, 31, size=(2, 1000, 16)))
    g, _ = oracle.score_cosine(K)
    w, _ = oracle.score_cosine_windowed(K, 1000)
    np.testing.assert_array_equal(g, w)
    w, mus = oracle.score_cosine_windowed(K, 300)  # windows 300, 300, 300, 100
    for j, t0 in enumerate(range(0, 1000, 300)):
        part, mu = oracle.score_cosine(K[:, t0:t0 + 300])
        np.testing.assert_array_equal(w[:, t0:t0 + 300], part)
        np.testing.assert_array_equal(mus[:, j], mu)


def test_range_and_nonfinite():
    rng = np.random.default_rng(9)
    K = int_bf16(rng.integers(-9, 10, size=(3, 200, 8)))
    s, _ = oracle.score_cosine(K)
    assert np.all(s >= -1e-15) and np.all(s <= 2.0 + 1e-15)
    bad = K.copy()
    bad[0, 3, 2] = 0x7F80  # +inf
    with pytest.raises(Exception):
        oracle.score_cosine(bad)
