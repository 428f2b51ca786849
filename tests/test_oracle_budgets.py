"""Pins for the oracle's RippleKV budget allocation ("RippleKV: Cross-Layer KV
Cache Allocation via Perturbation Propagation", sensitivity-guided budget
allocation: normalised sensitivities, multipliers r^s clipped to [1/gamma, gamma],
rescaled so the layer budgets sum to the global budget B) and of the ragged
top-k built on the per-slice select.  Independent of the oracle's code: closed
forms, invariances, the budget identity, bounds and monotonicity."""
import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import oracle


def test_two_layer_closed_form():
    # s^ = (0, 1): w = (1, r) when 1/gamma <= 1 and r <= gamma -> budgets B/(1+r), rB/(1+r)
    k = oracle.layer_budgets([0.2, 0.7], 4.0, 10.0, 1000, 10 ** 6)
    np.testing.assert_array_equal(k, [200, 800])
    # clipped at gamma: r = 16 > gamma = 2 -> w = (1, 2)
    k = oracle.layer_budgets([5.0, 9.0], 16.0, 2.0, 900, 10 ** 6)
    np.testing.assert_array_equal(k, [300, 600])
    # r = 1/4 < 1: the sensitive layer gets less; w = (1, 1/4) within [1/8, 8]
    k = oracle.layer_budgets([1.0, 3.0], 0.25, 8.0, 500, 10 ** 6)
    np.testing.assert_array_equal(k, [400, 100])


def test_uniform_sensitivity_or_r_one_is_uniform():
    for s, r in (([0.3] * 7, 8.0), (np.arange(7.0), 1.0)):
        k = oracle.layer_budgets(s, r, 4.0, 7 * 123 + 5, 10 ** 6)
        assert k.sum() == 7 * 123 + 5
        assert k.max() - k.min() <= 1
        np.testing.assert_array_equal(k, [124] * 5 + [123] * 2)  # remainder to the lower layers


def test_affine_invariance_of_the_normalisation():
    rng = np.random.default_rng(4)
    s = rng.exponential(1.0, 32)
    k0 = oracle.layer_budgets(s, 6.0, 3.0, 32 * 8192, 16384)
    for a, c in ((2.0, 0.0), (0.5, 10.0), (1e3, -7.0)):
        np.testing.assert_array_equal(oracle.layer_budgets(a * s + c, 6.0, 3.0, 32 * 8192, 16384), k0)


def test_capping_at_the_token_count():
    # one very sensitive layer would get more than S: it keeps S, the others share the rest
    s = [0.0, 0.0, 0.0, 1.0]
    k = oracle.layer_budgets(s, 100.0, 100.0, 250, 120)
    np.testing.assert_array_equal(k, [44, 43, 43, 120])
    # B = L * S keeps everything
    np.testing.assert_array_equal(oracle.layer_budgets(s, 100.0, 100.0, 480, 120), [120] * 4)
    np.testing.assert_array_equal(oracle.layer_budgets(s, 100.0, 100.0, 0, 120), [0] * 4)


@settings(max_examples=60, deadline=None)
@given(L=st.integers(1, 40), seed=st.integers(0, 10 ** 6), r=st.floats(0.1, 50.0),
       gamma=st.floats(1.0, 20.0), S=st.integers(1, 5000), frac=st.floats(0.0, 1.0))
def test_budget_identity_bounds_and_monotonicity(L, seed, r, gamma, S, frac):
    rng = np.random.default_rng(seed)
    s = rng.normal(0.0, 1.0, L)
    B = int(frac * L * S)
    k = oracle.layer_budgets(s, r, gamma, B, S)
    assert k.sum() == B and k.min() >= 0 and k.max() <= S
    # multipliers are monotone in s (r > 1 increasing, r < 1 decreasing), so are budgets
    order = np.argsort(s, kind="stable")
    ks = k[order]
    if r > 1:
        assert np.all(np.diff(ks) >= -1)
    elif r < 1:
        assert np.all(np.diff(ks) <= 1)
    # clipping bounds the disparity: uncapped budgets differ by at most gamma^2 (+ rounding)
    free = k[k < S]
    if free.size >= 2 and free.min() > 0 and B >= 50 * L:
        assert free.max() <= gamma ** 2 * free.min() + gamma ** 2 + 1


def test_invalid_arguments():
    with pytest.raises(Exception):
        oracle.layer_budgets([0.0, 1.0], 2.0, 0.5, 10, 10)   # gamma < 1
    with pytest.raises(Exception):
        oracle.layer_budgets([0.0, 1.0], 2.0, 2.0, 21, 10)   # B > L * S
    with pytest.raises(Exception):
        oracle.layer_budgets([0.0, np.nan], 2.0, 2.0, 5, 10)


def test_ragged_topk_is_per_slice_topk_packed():
    rng = np.random.default_rng(8)
    s = rng.normal(size=(5, 300)).astype(np.float32)
    ks = np.array([0, 1, 150, 299, 300])
    packed = oracle.topk_ragged(s, ks)
    assert packed.size == ks.sum()
    off = 0
    for g in range(5):
        part = packed[off:off + ks[g]]
        # brute force: the ks[g] largest, ties to the lower index (none here), ascending
        ref = np.sort(np.argsort(-s[g], kind="stable")[:ks[g]])
        np.testing.assert_array_equal(part, ref)
        off += ks[g]
