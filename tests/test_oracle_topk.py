"""Pins for the oracle's retention (top-k) and compaction (gather): a textbook
sort, brute-force dominance on tiny inputs and degenerate cases.  Sources:
ManifoldKV abstract and lay summary (the keys farthest from the centroid are
kept); OjaKV method details (top-k error scores kept at full rank)."""
import itertools

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import oracle


def textbook_topk(s, k):
    out = []
    for row in s:
        order = np.lexsort((np.arange(row.size), -row.astype(np.float64)))
        out.append(np.sort(order[:k]))
    return np.array(out, dtype=np.int32).reshape(len(s), k)


@settings(max_examples=60, deadline=None)
@given(G=st.integers(1, 3), S=st.integers(1, 60), seed=st.integers(0, 10**6),
       kind=st.sampled_from(["normal", "ties", "signed"]), data=st.data())
def test_matches_textbook_sort(G, S, seed, kind, data):
    import synth
    k = data.draw(st.integers(0, S))
    s = synth.random_scores(G, S, seed=seed, kind=kind).numpy()
    np.testing.assert_array_equal(oracle.topk(s, k), textbook_topk(s, k))


def test_bruteforce_dominance_tiny():
    # every kept token beats every evicted one under (score desc, index asc); exactly k kept
    rng = np.random.default_rng(7)
    for S in range(1, 8):
        for _ in range(20):
            s = rng.integers(0, 3, size=(1, S)).astype(np.float32)
            for k in range(S + 1):
                idx = oracle.topk(s, k)[0]
                kept = set(idx.tolist())
                assert len(kept) == k and list(idx) == sorted(kept)
                for a, b in itertools.product(kept, set(range(S)) - kept):
                    assert (s[0, a] > s[0, b]) or (s[0, a] == s[0, b] and a < b)


def test_degenerate_cases():
    s = np.full((2, 10), 3.5, np.float32)
    np.testing.assert_array_equal(oracle.topk(s, 4), [[0, 1, 2, 3]] * 2)
    np.testing.assert_array_equal(oracle.topk(s, 10), [list(range(10))] * 2)
    assert oracle.topk(s, 0).shape == (2, 0)
    # +0.0 and -0.0 are equal scores: index order decides
    z = np.array([[-0.0, 0.0, -0.0, 0.0]], np.float32)
    np.testing.assert_array_equal(oracle.topk(z, 2), [[0, 1]])
    with pytest.raises(ValueError):
        oracle.topk(s, 11)
    bad = s.copy()
    bad[1, 3] = np.nan
    with pytest.raises(ValueError):
        oracle.topk(bad, 3)


def test_strided_rows_ignore_padding():
    s = np.array([[1, 5, 2, 9, 9], [7, 0, 3, 9, 9]], np.float32)  # last 2 columns are padding
    np.testing.assert_array_equal(oracle.topk(s, 2, S=3), [[1, 2], [0, 2]])


def test_gather_is_index_select():
    rng = np.random.default_rng(5)
    X = rng.integers(0, 65536, size=(3, 50, 16), dtype=np.uint16)
    idx = np.sort(np.stack([rng.choice(50, 20, replace=False) for _ in range(3)]), axis=1).astype(np.int32)
    out = oracle.gather(X, idx)
    np.testing.assert_array_equal(out, np.take_along_axis(X, idx[:, :, None].astype(np.int64), axis=1))
    with pytest.raises(ValueError):
        oracle.gather(X, np.full((3, 1), 50, np.int32))


def test_keep_and_anchor_counts():
    # "drop 20%, keep 3277" of 4096; 50% of 16384; 25% of 65536; 5% anchors (ceil)
    assert oracle.keep_count(4096, 20) == 3277
    assert oracle.keep_count(16384, 50) == 8192
    assert oracle.keep_count(65536, 25) == 49152
    assert oracle.n_anchors(32768) == 1639
    assert oracle.n_anchors(131072) == 6554
    assert oracle.n_anchors(131072 + 32 * 8) == 6567
