"""Pins of the oracle's top-k and candidate block selection.

Top-k definition: "DeepSeek V4.1" page, class Indexer, forward (top-k of
min(index_topk, end_pos//ratio), re-sorted by position, -1 where the index
is not below compress_lens, offset added).  Short-context closed form: the
vLLM attention.py page, _fill_short_context_topk_indices.  Block selection:
"DeepSeek V4.1" page (select_candidate_blocks call) and the "Module compress"
page (select_candidate_blocks), whose body is not given; the block-max
reading is chosen here (the pages leave the block score open).
"""
import numpy as np
import pytest

import oracle


def _rows(rng, R, T, nvals):
    """Scores drawn from a few values so that ties are frequent; some -inf
    and some -0.0."""
    vals = np.concatenate([rng.standard_normal(nvals).astype(np.float32), [0.0, -0.0, -np.inf]])
    return vals[rng.integers(0, len(vals), size=(R, T))].astype(np.float32)


@pytest.mark.parametrize("seed", range(6))
def test_topk_matches_lexsort_bruteforce(seed):
    rng = np.random.default_rng(seed)
    R, T = 13, int(rng.integers(1, 300))
    s = _rows(rng, R, T, nvals=int(rng.integers(1, 40)))
    cl = rng.integers(0, T + 3, size=R).astype(np.int32)
    for k in (1, 3, T // 2 + 1, T, T + 5):
        off = int(rng.integers(-5, 1000))
        got = oracle.topk(s, cl, k, off)
        for r in range(R):
            assert np.array_equal(got[r], oracle.topk_bruteforce(s[r], int(cl[r]), k, off))


def test_topk_invariants():
    rng = np.random.default_rng(7)
    R, T, k, off = 50, 1000, 64, 17
    s = rng.standard_normal((R, T)).astype(np.float32)
    cl = rng.integers(0, T + 1, size=R).astype(np.int32)
    out = oracle.topk(s, cl, k, off)
    assert out.shape == (R, min(k, T))
    for r in range(R):
        o = out[r]
        valid = o[o != -1]
        n_neg = int((o == -1).sum())
        assert n_neg == max(0, min(k, T) - int(cl[r]))  # -1 only when too few reachable
        assert np.all(o[: len(valid)] == valid)  # -1 only at the tail
        assert np.all(np.diff(valid) > 0)  # position order
        assert np.all((valid - off >= 0) & (valid - off < cl[r]))
        # every selected score >= every unselected reachable score
        sel = valid - off
        rest = np.setdiff1d(np.arange(min(cl[r], T)), sel)
        if len(sel) and len(rest):
            assert s[r, sel].min() >= s[r, rest].max()


def test_short_context_closed_form():
    """T <= index_topk: every position is kept; out[i] = i + offset for
    i < compress_lens, else -1 (the vLLM short-context fill, plus offset as
    the Indexer adds it)."""
    rng = np.random.default_rng(8)
    for T, k, off in ((5, 8, 0), (512, 512, 3), (100, 2048, 9)):
        s = rng.standard_normal((4, T)).astype(np.float32)
        cl = np.array([0, 1, T // 2, T], np.int32)
        out = oracle.topk(s, cl, k, off)
        for r in range(4):
            exp = [i + off if i < cl[r] else -1 for i in range(T)]
            assert list(out[r]) == exp


def test_ties_take_lowest_position_and_signed_zero_ties():
    s = np.array([[1.0, 2.0, 2.0, 0.0, -0.0, 2.0, 0.0]], np.float32)
    cl = np.array([7], np.int32)
    assert list(oracle.topk(s, cl, 2)[0]) == [1, 2]
    assert list(oracle.topk(s, cl, 4)[0]) == [0, 1, 2, 5]
    assert list(oracle.topk(s, cl, 5)[0]) == [0, 1, 2, 3, 5]  # -0 at 4 ties +0 at 3
    assert list(oracle.topk(s, cl, 6)[0]) == [0, 1, 2, 3, 4, 5]


def test_topk_empty_rows():
    s = np.zeros((3, 0), np.float32)
    out = oracle.topk(s, np.zeros(3, np.int32), 16)
    assert out.shape == (3, 0)


@pytest.mark.parametrize("seed", range(4))
def test_select_blocks_matches_bruteforce(seed):
    rng = np.random.default_rng(100 + seed)
    R, T = 9, int(rng.integers(1, 700))
    cbs = int(rng.choice([1, 7, 16, 64]))
    s = _rows(rng, R, T, nvals=50)
    s[np.isneginf(s)] = 0.0  # scores below cl are finite
    cl = rng.integers(0, T + 1, size=R).astype(np.int32)
    for ctb in (1, 3, 1000):
        ids = oracle.select_blocks(s, cl, ctb, cbs)
        for r in range(R):
            assert np.array_equal(ids[r], oracle.select_blocks_bruteforce(s[r], int(cl[r]), ctb,
                                                                          cbs))


def test_select_all_blocks_when_ctb_covers_width():
    rng = np.random.default_rng(9)
    T, cbs = 1000, 128
    s = rng.standard_normal((3, T)).astype(np.float32)
    cl = np.array([1000, 300, 0], np.int32)
    ids = oracle.select_blocks(s, cl, 64, cbs)
    nb = 8
    for r in range(3):
        reach = (int(cl[r]) + cbs - 1) // cbs
        assert list(ids[r]) == [j if j < reach else -1 for j in range(nb)]
