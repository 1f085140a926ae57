"""GPU parity of the T-split top-k: idx_topk_pairs on each slice of the rows
(positions bit-exact against oracle.topk_pairs, scores equal to the slice's
scores at them) and idx_merge_topk of the slices' lists, bit-exact against
oracle.topk of the whole rows.  Definition: "DeepSeek V4.1" page, class
Indexer, forward (top-k, position re-sort, -1 and offset); the merge is exact
because a position in a row's top k is in its slice's top k.

Cases: the long-row decode shape (4 rows of 262144 positions in 8 slices of
32768, k 2048), rows ranked by the chunked path inside a slice (slices wider
than 32768 without a histogram), the longest lists (16 x 2048 pairs), lists
shorter than a wave (k 5), k beyond a slice's width, k >= T, uneven slices,
compress_lens in every slice, at 0 and at T, scores with many ties (across
slice edges), -0 and +0, -inf; and lists that are not top-k lists (fewer
valid pairs than k_out); and 12 seeded random shapes."""
import numpy as np
import pytest

import oracle

from gpu_util import dev, host, say, sync, torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def idx():
    import sparse_attention_top_fp4_amd as m
    m.load_library()
    return m


def _scores(rng, R, T, nvals):
    if nvals == 0:
        return rng.standard_normal((R, T)).astype(np.float32)
    vals = np.concatenate([rng.standard_normal(nvals).astype(np.float32), [0.0, -0.0, -np.inf]])
    return vals[rng.integers(0, len(vals), size=(R, T))].astype(np.float32)


def _slices(T, G, even, rng):
    if even:
        w = T // G
        return [(g * w, w if g < G - 1 else T - g * w) for g in range(G)]
    cuts = np.sort(rng.integers(1, T, size=G - 1))
    e = np.concatenate([[0], cuts, [T]]).astype(int)
    return [(int(e[g]), int(e[g + 1] - e[g])) for g in range(G)]


MERGE_CASES = [
    # (seed, R, T, G, even, k, nvals (0: no ties), compress_lens or None)
    (201, 4, 262144, 8, True, 2048, 0, [262144, 200000, 20000, 1000]),  # long-row decode
    (202, 5, 3000, 3, False, 200, 7, None),                              # many ties, uneven
    (203, 3, 70000, 2, True, 2048, 0, [70000, 36000, 30000]),            # chunked slices
    (204, 2, 65536, 16, True, 2048, 20, [65536, 40000]),                 # 16 x 2048 pairs
    (205, 6, 100, 4, False, 5, 3, None),                                 # lists of 5
    (206, 4, 1000, 4, True, 300, 50, [1000, 999, 600, 301]),             # k > slice width
    (207, 3, 500, 3, False, 600, 10, [500, 250, 0]),                     # k >= T
    (208, 7, 9000, 5, False, 1024, 2, None),                             # heavy ties
]


@pytest.mark.parametrize("case", MERGE_CASES, ids=[str(c[0]) for c in MERGE_CASES])
def test_merge_of_slices_matches_row_topk(idx, case):
    seed, R, T, G, even, k, nvals, cl_over = case
    t = torch()
    rng = np.random.default_rng(seed)
    s = _scores(rng, R, T, nvals)
    cl = (np.array(cl_over, np.int32) if cl_over is not None
          else rng.integers(0, T + 2, size=R).astype(np.int32))
    slices = _slices(T, G, even, rng)
    n = max(min(k, w) for _, w in slices)
    offset = int(rng.integers(0, 500))
    say("merge", seed, R, T, G, k, "slices", slices[:3], "...")
    sd, cld = dev(s), dev(cl)
    pos = t.full((G, R, n), -1, dtype=t.int32, device="cuda")
    sco = t.full((G, R, n), float("-inf"), dtype=t.float32, device="cuda")
    for g, (start, w) in enumerate(slices):
        kl = min(k, w)
        po = t.empty((R, kl), dtype=t.int32, device="cuda")
        so = t.empty((R, kl), dtype=t.float32, device="cuda")
        assert idx.idx_topk_pairs(sd, start, w, cld, k, po, so) == kl
        pos[g, :, :kl] = po
        sco[g, :, :kl] = so
        sync()
        wp, ws = oracle.topk_pairs(s, cl, k, start, w)
        assert np.array_equal(host(po), wp), ("pairs", g)
        assert np.array_equal(host(so).view(np.uint32), ws.view(np.uint32)), ("pair scores", g)
    kout = min(k, T)
    out = t.full((R, kout + 3), -7, dtype=t.int32, device="cuda")
    assert idx.idx_merge_topk(pos, sco, cld, T, k, offset, out) == kout
    sync()
    got = host(out)
    want = oracle.topk(s, cl, k, offset)
    assert np.array_equal(got[:, :kout], want)
    assert (got[:, kout:] == -7).all()  # nothing past k_out is written
    # the oracle's merge of the GPU's lists agrees too
    assert np.array_equal(oracle.merge_topk(host(pos), host(sco), cl, T, k, offset), want)


def test_merge_with_fewer_valid_pairs_than_k(idx):
    t = torch()
    # ascending lists holding 3 valid pairs for k_out 5 (compress_lens 20 > 5),
    # and a row whose lists are all -1
    pos = np.array([[[2, 7, -1], [-1, -1, -1]], [[11, -1, -1], [-1, -1, -1]]], np.int32)
    sc = np.array([[[4.0, 1.0, -np.inf], [0, 0, 0]], [[0.5, -np.inf, -np.inf], [0, 0, 0]]],
                  np.float32)
    cl = np.array([20, 20], np.int32)
    say("merge guard")
    out = t.empty((2, 5), dtype=t.int32, device="cuda")
    idx.idx_merge_topk(dev(pos), dev(sc), dev(cl), 20, 5, 3, out)
    sync()
    got = host(out)
    assert got.tolist() == [[5, 10, 14, -1, -1], [-1, -1, -1, -1, -1]]
    assert np.array_equal(got, oracle.merge_topk(pos, sc, cl, 20, 5, 3))


def test_merge_rows_at_or_below_k_out_take_the_closed_form(idx):
    t = torch()
    R, T, k = 3, 4000, 100
    rng = np.random.default_rng(209)
    pos = t.full((2, R, 100), -1, dtype=t.int32, device="cuda")  # contents unused
    sco = t.zeros((2, R, 100), dtype=t.float32, device="cuda")
    cl = np.array([100, 7, 0], np.int32)
    say("merge closed form")
    out = t.empty((R, k), dtype=t.int32, device="cuda")
    idx.idx_merge_topk(pos, sco, dev(cl), T, k, 9, out)
    sync()
    s = rng.standard_normal((R, T)).astype(np.float32)
    assert np.array_equal(host(out), oracle.topk(s, cl, k, 9))


@pytest.mark.parametrize("seed", range(12))
def test_merge_fuzz(idx, seed):
    """Seeded random shapes: rows, width, slices (uneven), k on both sides of
    the slices' and the rows' widths, compress_lens in [-2, T + 3], offsets of
    both signs, ties."""
    t = torch()
    rng = np.random.default_rng(300 + seed)
    R = int(rng.integers(1, 7))
    T = int(rng.integers(2, 20000))
    G = int(rng.integers(1, min(9, T) + 1))
    k = int(rng.integers(1, 3000))
    slices = _slices(T, G, False, rng) if G > 1 else [(0, T)]
    n = max(min(k, w) for _, w in slices)  # G * n <= 9 * 2999: within the merge's 32768
    s = _scores(rng, R, T, int(rng.integers(0, 40)))
    cl = rng.integers(-2, T + 4, size=R).astype(np.int32)
    offset = int(rng.integers(-1000, 1000))
    say("merge fuzz", seed, R, T, G, k, n)
    sd, cld = dev(s), dev(cl)
    pos = t.full((G, R, n), -1, dtype=t.int32, device="cuda")
    sco = t.full((G, R, n), float("-inf"), dtype=t.float32, device="cuda")
    for g, (start, w) in enumerate(slices):
        kl = min(k, w)
        po = t.empty((R, kl), dtype=t.int32, device="cuda")
        so = t.empty((R, kl), dtype=t.float32, device="cuda")
        idx.idx_topk_pairs(sd, start, w, cld, k, po, so)
        pos[g, :, :kl] = po
        sco[g, :, :kl] = so
    kout = min(k, T)
    out = t.empty((R, kout), dtype=t.int32, device="cuda")
    idx.idx_merge_topk(pos, sco, cld, T, k, offset, out)
    sync()
    assert np.array_equal(host(out), oracle.topk(s, cl, k, offset))
