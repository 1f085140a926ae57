"""GPU parity of the paged key cache entry points ([VLLM,
DeepseekV4IndexerCache]: pages of 64 compressed positions reached through a
per-sequence block table).  The rows of a contiguous cache are scattered
over a larger page pool (padded page stride, pages out of order); table
entries the call must not use hold ids outside the pool.  Scores must be
bit-identical to the oracle's and to the contiguous path's, histograms
equal, indices and published rows bit-exact."""
import numpy as np
import pytest

import oracle
from sparse_attention_top_fp4_amd.inputs import YARN, normal_bf16, small_case

from gpu_util import bits, dev, fp4_cache, host, say, sync, torch

pytestmark = pytest.mark.gpu

PAGE = 64
PAGE_STRIDE = PAGE * 68 + 128  # padded pages


@pytest.fixture(scope="module")
def idx():
    import sparse_attention_top_fp4_amd as m
    m.load_library()
    return m


def _paginate(kc_dev, used_pages, seed):
    """Scatter a contiguous device cache [B, T, 68] into a page pool: returns
    (pages [n_pages, PAGE_STRIDE] uint8, block_table [B, ceil(T/64)] int32).
    Logical pages j >= used_pages[b] of sequence b get an id past the pool."""
    t = torch()
    B, T, _ = kc_dev.shape
    npg = (T + PAGE - 1) // PAGE
    rng = np.random.default_rng(seed)
    n_pages = B * npg + 5
    perm = rng.permutation(n_pages)
    pages = t.zeros((n_pages, PAGE_STRIDE), dtype=t.uint8, device="cuda")
    bt = np.full((B, npg), n_pages + 7, np.int32)
    k = 0
    for b in range(B):
        for j in range(npg):
            p = int(perm[k])
            k += 1
            rows = kc_dev[b, j * PAGE:(j + 1) * PAGE].reshape(-1)
            pages[p, :rows.numel()] = rows
            if j < used_pages[b]:
                bt[b, j] = p
    return pages, dev(bt)


@pytest.mark.parametrize("B,S,T,sp", [(3, 1, 5000, None), (1, 24, 3000, 1999)])
def test_score_paged_matches_oracle_and_contiguous(idx, B, S, T, sp):
    t = torch()
    say("score paged", B, S, T, sp)
    c = small_case(90 + S, B, S, 64, T, start_pos=sp)
    if S == 1:
        c["cl"][:] = np.array([T, 4097, 63][:B], np.int32)
    R = B * S
    kc_ref, _ = oracle.fp4_quant_rows(c["k"])
    ref, inexact = oracle.score(c["q"], c["w"], kc_ref, B, S, 64, T, c["cl"])
    assert inexact == 0
    kc = fp4_cache(c["k"])
    cl_seq = c["cl"].reshape(B, S).max(axis=1)
    pages, bt = _paginate(kc, [(int(x) + PAGE - 1) // PAGE for x in cl_seq], 5 + S)
    sc = t.full((R, T), float("nan"), dtype=t.float32, device="cuda")
    hist = t.zeros((R, 2048), dtype=t.int32, device="cuda")
    idx.idx_score_paged(dev(c["q"]), dev(c["w"]), pages, bt, B, S, T, dev(c["cl"]), sc,
                        key_hist=hist)
    sc2 = t.full((R, T), float("nan"), dtype=t.float32, device="cuda")
    hist2 = t.zeros((R, 2048), dtype=t.int32, device="cuda")
    idx.idx_score(dev(c["q"]), dev(c["w"]), kc, B, S, T, dev(c["cl"]), sc2, key_hist=hist2)
    sync()
    g, g2 = host(sc), host(sc2)
    for r in range(R):
        n = int(c["cl"][r])
        assert np.array_equal(bits(g[r, :n]), bits(ref[r, :n])), r
        assert np.array_equal(bits(g[r, :n]), bits(g2[r, :n])), r
    assert np.array_equal(host(hist), host(hist2))


@pytest.mark.parametrize("B,S,T,sp,k,with_scores", [
    (2, 16, 6000, 16380, 2048, True),   # prefill rows ranked in two layouts
    (3, 1, 8192, None, 2048, False),    # decode at the widest fused row
    (1, 40, 3000, 0, 5, False),         # short rows: cl <= k kept in closed form
])
def test_score_topk_paged_matches_oracle(idx, B, S, T, sp, k, with_scores):
    t = torch()
    say("score+topk paged", B, S, T, sp, k, with_scores)
    c = small_case(95 + S, B, S, 64, T, start_pos=sp)
    R = B * S
    kc_ref, _ = oracle.fp4_quant_rows(c["k"])
    ref, _ = oracle.score(c["q"], c["w"], kc_ref, B, S, 64, T, c["cl"])
    kc = fp4_cache(c["k"])
    cl_seq = c["cl"].reshape(B, S).max(axis=1)
    pages, bt = _paginate(kc, [(int(x) + PAGE - 1) // PAGE for x in cl_seq], 9 + S)
    kout = min(k, T)
    out = t.full((R, kout + 1), -7, dtype=t.int32, device="cuda")
    sc = t.full((R, T), float("nan"), dtype=t.float32, device="cuda") if with_scores else None
    idx.idx_score_topk_paged(dev(c["q"]), dev(c["w"]), pages, bt, B, S, T, dev(c["cl"]), k, 3,
                             out, scores=sc)
    out2 = t.full((R, kout + 1), -7, dtype=t.int32, device="cuda")
    idx.idx_score_topk(dev(c["q"]), dev(c["w"]), kc, B, S, T, dev(c["cl"]), k, 3, out2)
    sync()
    got = host(out)
    assert np.array_equal(got[:, :kout], oracle.topk(ref, c["cl"], k, 3))
    assert np.array_equal(got, host(out2))
    assert np.all(got[:, kout:] == -7)
    if with_scores:
        g = host(sc)
        for r in range(R):
            n = int(c["cl"][r])
            assert np.array_equal(bits(g[r, :n]), bits(ref[r, :n])), r


@pytest.mark.parametrize("mode", ["decode", "prefill"])
def test_publish_paged_matches_oracle(idx, mode):
    t = torch()
    say("publish paged", mode)
    rng = np.random.default_rng(61)
    B, din, tcap = 3, 512, 300
    G = 1 if mode == "decode" else 37
    start_pos = 4 * 250 - 1 if mode == "decode" else 0
    latent = normal_bf16(rng, (B, G, din))
    wk = normal_bf16(rng, (128, din), std=0.02)
    gamma = (1.0 + 0.1 * rng.standard_normal(128)).astype(np.float32)
    P = 1200
    cs = oracle.yarn_cos_sin(P, 64, YARN["theta"], YARN["factor"], YARN["orig_len"],
                             YARN["beta_fast"], YARN["beta_slow"])
    kc0 = rng.integers(0, 256, size=(B, tcap, 68), dtype=np.uint8)
    kc_ref = kc0.copy()
    oracle.publish(latent, wk, gamma, cs, start_pos, 4, 1e-6, kc_ref)
    npg = (tcap + PAGE - 1) // PAGE
    # every page of sequences 0 and 1 is mapped; sequence 2 maps none, so its
    # row is not written anywhere
    pages, bt = _paginate(dev(kc0), [npg, npg, 0], 71)
    before = host(pages).copy()
    idx.idx_publish_keys_paged(dev(latent), dev(wk), dev(gamma), dev(cs), start_pos, 4, 1e-6,
                               pages, bt, tcap)
    sync()
    pg, table = host(pages), host(bt)
    for b in range(2):
        got = np.concatenate([pg[table[b, j], :PAGE * 68].reshape(PAGE, 68) for j in range(npg)])
        assert np.array_equal(got[:tcap], kc_ref[b]), b
    # sequence 2's pages are untouched, and so is every unmapped page
    mapped = set(table[:2].reshape(-1).tolist())
    for p in range(pg.shape[0]):
        if p not in mapped:
            assert np.array_equal(pg[p], before[p]), p


def test_score_paged_candidates_match_oracle(idx):
    """Level two on pages: candidate blocks of 128 positions (ids out of range
    skipped), scores bit-identical to the oracle and to the contiguous path;
    a candidate page whose id is outside the pool scores as zero rows."""
    t = torch()
    say("score paged candidates")
    B, T, cbs = 2, 5000, 128
    c = small_case(97, B, 1, 64, T)
    c["cl"][:] = np.array([T, 3001], np.int32)
    cand = np.array([[0, 7, 38, 39, -1, 500], [2, 3, 23, 30, 31, 1]], np.int32)
    kc_ref, _ = oracle.fp4_quant_rows(c["k"])
    ref, _ = oracle.score(c["q"], c["w"], kc_ref, B, 1, 64, T, c["cl"], cand=cand, cbs=cbs)
    kc = fp4_cache(c["k"])
    pages, bt = _paginate(kc, [(int(x) + PAGE - 1) // PAGE for x in c["cl"]], 97)
    sc = t.full((B, T), float("nan"), dtype=t.float32, device="cuda")
    hist = t.zeros((B, 2048), dtype=t.int32, device="cuda")
    idx.idx_score_paged(dev(c["q"]), dev(c["w"]), pages, bt, B, 1, T, dev(c["cl"]), sc,
                        cand_blocks=dev(cand), cand_block_size=cbs, key_hist=hist)
    sc2 = t.full((B, T), float("nan"), dtype=t.float32, device="cuda")
    hist2 = t.zeros((B, 2048), dtype=t.int32, device="cuda")
    idx.idx_score(dev(c["q"]), dev(c["w"]), kc, B, 1, T, dev(c["cl"]), sc2,
                  cand_blocks=dev(cand), cand_block_size=cbs, key_hist=hist2)
    sync()
    assert np.array_equal(bits(host(sc)), bits(ref))
    assert np.array_equal(bits(host(sc)), bits(host(sc2)))
    assert np.array_equal(host(hist), host(hist2))
    # sequence 1's page 46 (positions 2944..3007, inside candidate block 23)
    # made invalid: its scored positions become relu(0) sums, +0
    bt_bad = host(bt).copy()
    bt_bad[1, 46] = pages.shape[0] + 3
    idx.idx_score_paged(dev(c["q"]), dev(c["w"]), pages, dev(bt_bad), B, 1, T, dev(c["cl"]), sc,
                        cand_blocks=dev(cand), cand_block_size=cbs)
    sync()
    g = host(sc)
    assert np.all(g[1, 2944:3001] == 0.0) and not np.any(np.signbit(g[1, 2944:3001]))
    assert np.array_equal(bits(g[1, 2940:2944]), bits(ref[1, 2940:2944]))
    assert np.array_equal(bits(g[0]), bits(ref[0]))
