"""Pins of the oracle's T-split top-k: each slice's top-k as (position,
score) pairs (oracle.topk_pairs) and the merge of the slices' lists
(oracle.merge_topk).

Definition: "DeepSeek V4.1" page, class Indexer, forward (top-k of the
masked scores, re-sorted by position, -1 where the index is not below
compress_lens, offset added).  The merge rests on a property of that
definition: a position in a row's top k is beaten by fewer than k positions
of the row, hence of its own slice, so it is in its slice's top k.  The pins
check the merge against oracle.topk of the whole row (itself pinned by the
lexsort brute force in test_oracle_topk.py) and against hand-worked rows.
"""
import numpy as np
import pytest

import oracle


def _rows(rng, R, T, nvals):
    """Scores drawn from a few values so that ties are frequent (across slice
    edges too); some -inf and some -0.0."""
    vals = np.concatenate([rng.standard_normal(nvals).astype(np.float32), [0.0, -0.0, -np.inf]])
    return vals[rng.integers(0, len(vals), size=(R, T))].astype(np.float32)


def _split(T, G, rng):
    """G consecutive slices covering [0, T), uneven, some possibly empty."""
    cuts = np.sort(rng.integers(0, T + 1, size=G - 1))
    edges = np.concatenate([[0], cuts, [T]]).astype(int)
    return [(int(edges[g]), int(edges[g + 1] - edges[g])) for g in range(G)]


def _merge_slices(s, cl, k, slices, offset):
    R = s.shape[0]
    n = max(min(k, w) for _, w in slices) if slices else 0
    pos = np.full((len(slices), R, n), -1, np.int32)
    sc = np.full((len(slices), R, n), -np.inf, np.float32)
    for g, (start, w) in enumerate(slices):
        p, v = oracle.topk_pairs(s, cl, k, start, w)
        pos[g, :, :p.shape[1]] = p
        sc[g, :, :p.shape[1]] = v
    return oracle.merge_topk(pos, sc, cl, s.shape[1], k, offset)


@pytest.mark.parametrize("seed", range(8))
def test_merge_of_slice_lists_equals_row_topk(seed):
    rng = np.random.default_rng(100 + seed)
    R, T = 9, int(rng.integers(2, 600))
    s = _rows(rng, R, T, nvals=int(rng.integers(1, 30)))
    # compress_lens in every part of the row: 0, below k, inside any slice, T, beyond T
    cl = rng.integers(0, T + 3, size=R).astype(np.int32)
    cl[0], cl[1] = T, 0
    for G in (1, 2, 3, 5):
        slices = _split(T, G, rng)
        for k in (1, 4, T // 3 + 1, T - 1 if T > 1 else 1, T + 2):
            off = int(rng.integers(0, 1000))
            want = oracle.topk(s, cl, k, off)
            got = _merge_slices(s, cl, k, slices, off)
            assert np.array_equal(got, want), (G, k, slices)


def test_pairs_are_the_slice_topk_with_row_positions():
    rng = np.random.default_rng(5)
    R, T = 6, 300
    s = _rows(rng, R, T, 12)
    cl = np.array([300, 250, 120, 100, 0, 180], np.int32)
    pos, sc = oracle.topk_pairs(s, cl, 40, 100, 100)
    for r in range(R):
        c_loc = min(max(int(cl[r]) - 100, 0), 100)
        want = oracle.topk_bruteforce(s[r, 100:200], c_loc, 40, 100)
        assert np.array_equal(pos[r], want)
        for j, p in enumerate(pos[r]):
            if p < 0:
                assert sc[r, j] == -np.inf
            else:
                assert sc[r, j] == s[r, p] and p < cl[r]


def test_hand_worked_tie_across_the_slice_edge():
    # row [1, 3, 2 | 3, 1, 5]: the two 3s sit in different slices
    s = np.array([[1, 3, 2, 3, 1, 5]], np.float32)
    slices = [(0, 3), (3, 3)]
    cases = [
        (6, 2, [1, 5]),        # 5, then the 3 at the lower position
        (6, 3, [1, 3, 5]),     # both 3s
        (6, 4, [1, 2, 3, 5]),  # then the 2
        (5, 2, [1, 3]),        # position 5 masked: the two 3s
        (2, 4, [0, 1, -1, -1]),  # compress_lens 2 <= k_out: the closed form
    ]
    for c, k, want in cases:
        cl = np.array([c], np.int32)
        got = _merge_slices(s, cl, k, slices, 0)
        assert got[0].tolist() == want, (c, k)
        assert oracle.topk(s, cl, k, 0)[0].tolist() == want
    # with an offset
    got = _merge_slices(s, np.array([6], np.int32), 3, slices, 100)
    assert got[0].tolist() == [101, 103, 105]


def test_merge_matches_lexsort_bruteforce_tiny():
    rng = np.random.default_rng(11)
    for _ in range(40):
        T = int(rng.integers(1, 20))
        s = _rows(rng, 1, T, int(rng.integers(1, 5)))
        cl = np.array([int(rng.integers(0, T + 2))], np.int32)
        k = int(rng.integers(1, T + 3))
        slices = _split(T, int(rng.integers(1, 4)), rng)
        got = _merge_slices(s, cl, k, slices, 7)
        assert np.array_equal(got[0], oracle.topk_bruteforce(s[0], int(cl[0]), k, 7))


def test_merge_with_fewer_valid_pairs_than_k():
    # lists that are not top-k lists: 3 valid pairs for k_out 5 with
    # compress_lens past k_out -> the valid ones by position, then -1
    pos = np.array([[[2, 7, -1]], [[11, -1, -1]]], np.int32)   # [G=2][R=1][n=3]
    sc = np.array([[[4.0, 1.0, -np.inf]], [[0.5, -np.inf, -np.inf]]], np.float32)
    got = oracle.merge_topk(pos, sc, np.array([20], np.int32), 20, 5, 0)
    assert got[0].tolist() == [2, 7, 11, -1, -1]
