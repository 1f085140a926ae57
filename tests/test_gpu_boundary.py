"""The top-k calls against a score histogram that does not belong to their
scores: a histogram filled twice (a top-k call skipped, or a NULL passed to
one), one filled by another call, or arbitrary counts.  Every top-k path
(rows of one workgroup, split rows over two kernels, the chunked path,
level-two candidate rows) checks the histogram's total against the row's
reachable count and, when it differs, ranks the row from its scores alone:
the indices must still equal the oracle's top-k ("DeepSeek V4.1" page, class
Indexer, forward: the final topk, sort by position, -1 and offset), and the
call must still leave the histogram zeroed."""
import numpy as np
import pytest

import oracle
from sparse_attention_top_fp4_amd.inputs import small_case

from gpu_util import dev, fp4_cache, host, say, sync, torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def idx():
    import sparse_attention_top_fp4_amd as m
    m.load_library()
    return m


STALE_CASES = [
    # (seed, B, T, candidate blocks, cbs, k, how the histogram goes wrong, path)
    (301, 3, 5000, None, 0, 2048, "double", "auto"),     # rows, 256 threads
    (302, 2, 30000, None, 0, 2048, "skipped", "auto"),   # rows, 1024 threads
    (303, 2, 40000, None, 0, 2048, "double", "auto"),    # split rows
    (304, 1, 70001, None, 0, 2048, "garbage", "auto"),   # split rows, ragged
    (305, 2, 9000, None, 0, 2048, "other", "auto"),      # rows: another row's counts
    (306, 2, 9000, None, 0, 2048, "double", "chunked"),  # chunked path
    (307, 2, 20000, [list(range(0, 128, 2)), list(range(1, 128, 2))], 128, 2048, "double",
     "auto"),                                            # level-two candidate rows
    (308, 2, 40000, None, 0, 2048, "garbage", "auto"),   # split, counts above T
]


@pytest.mark.parametrize("case", STALE_CASES)
def test_topk_with_stale_histogram(idx, case, monkeypatch):
    t = torch()
    seed, B, T, cand_rows, cbs, k, how, path = case
    if path == "chunked":
        monkeypatch.setenv("IDX_TOPK_PATH", "chunked")
    say("topk with a stale histogram", seed, B, T, cbs, k, how, path)
    c = small_case(seed, B, 1, 64, T)
    cl = c["cl"].copy()
    cl[0] = T - 17  # a row that does not see its whole cache
    kc_ref, _ = oracle.fp4_quant_rows(c["k"])
    cand = None if cand_rows is None else np.array(cand_rows, np.int32)
    ref, _ = oracle.score(c["q"], c["w"], kc_ref, B, 1, 64, T, cl, cand=cand, cbs=cbs)
    kc = fp4_cache(c["k"])
    sc = t.empty((B, T), dtype=t.float32, device="cuda")
    hist = t.empty((B, 2048), dtype=t.int32, device="cuda")
    idx.idx_clear_key_hist(hist)
    q, w, cld = dev(c["q"]), dev(c["w"]), dev(cl)
    cd = None if cand is None else dev(cand)

    def score(lens=cld, h=hist):
        idx.idx_score(q, w, kc, B, 1, T, lens, sc, cand_blocks=cd, cand_block_size=cbs,
                      key_hist=h)

    kout = min(k, T)
    out = t.full((B, kout), -7, dtype=t.int32, device="cuda")

    def topk(h):
        if cd is None:
            return idx.idx_topk(sc, T, cld, k, 3, out, key_hist=h)
        return idx.idx_topk_candidates(sc, T, cld, cd, cbs, k, 3, out, key_hist=h)

    if how == "double":      # two score calls into one histogram
        score()
        score()
    elif how == "skipped":   # a top-k given no histogram leaves it filled
        score()
        assert topk(None) == kout
        score()
    elif how == "other":     # counts of shorter rows
        score(lens=dev(np.full(B, T // 3, np.int32)))
        hist_other = hist.clone()
        idx.idx_clear_key_hist(hist)
        score(h=None)
        hist.copy_(hist_other)
    else:                    # arbitrary counts
        score(h=None)
        rng = np.random.default_rng(seed)
        hist.copy_(dev(rng.integers(0, 60, size=(B, 2048)).astype(np.int32)))
    assert topk(hist) == kout
    sync()
    assert np.array_equal(host(out), oracle.topk(ref, cl, k, 3))
    assert not host(hist).any()
