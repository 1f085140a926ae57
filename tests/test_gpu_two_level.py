"""GPU parity of idx_score_select_blocks, the level-one pass of the
two-level indexer: the scores (bit-identical to the oracle's below
compress_lens), the score histogram (exact counts of the scored positions)
and the selected block ids (bit-exact against the oracle's block select on
its own scores).  Cases take the single-launch form (block maxima from the
score launch, one wave per row ranks them) and both two-call forms (blocks
that straddle score chunks; more blocks than one wave ranks), with rows whose
compress_lens is T, a part of T, 1 and 0, decode and prefill rows, and 32
and 64 heads.  idx_score_topk_candidates, the level-two pass: slot scores
bit-identical to the oracle's scores at the slots' positions, indices and
the histogram's reset equal to idx_score + idx_topk_candidates, over
ascending lists with skipped ids (negative, past the row's blocks) in
between, rows with compress_lens below
the blocks, short lists (fewer finite candidates than k) and k >= T."""
import numpy as np
import pytest

import oracle
from sparse_attention_top_fp4_amd.inputs import small_case

from gpu_util import bits, dev, fp4_cache, host, say, sync, torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def idx():
    import sparse_attention_top_fp4_amd as m
    m.load_library()
    return m


def _counted_hist(scores_rows, cl, T):
    out = np.zeros((scores_rows.shape[0], 2048), np.int64)
    for r in range(scores_rows.shape[0]):
        n = max(0, min(int(cl[r]), T))
        v = scores_rows[r, :n].astype(np.float32)
        v = np.where(v == 0.0, np.float32(0.0), v)
        u = v.view(np.uint32)
        key = np.where(u & 0x80000000, ~u, u | 0x80000000).astype(np.uint32)
        out[r] = np.bincount(key >> 21, minlength=2048)
    return out


CASES = [
    # (seed, B, S, H, T, start_pos, cbs, ctb, cl override)
    (131, 4, 1, 64, 65536, None, 128, 64, [65536, 40000, 1, 0]),  # one launch + wave select
    (132, 2, 1, 32, 20000, None, 128, 16, None),                  # 32 heads, ragged last block
    (133, 1, 16, 64, 4096, 8000, 64, 8, None),                     # prefill rows, cl ~ 2000
    (134, 3, 1, 64, 30000, None, 100, 20, None),                   # blocks straddle chunks: two calls
    (135, 2, 1, 64, 200000, None, 128, 64, None),                  # 1563 blocks: two calls
]


@pytest.mark.parametrize("case", CASES)
def test_score_select_blocks_matches_oracle(idx, case):
    t = torch()
    seed, B, S, H, T, sp, cbs, ctb, cl = case
    say("score+select", case[:8])
    c = small_case(seed, B, S, H, T, start_pos=sp)
    if cl is not None:
        c["cl"] = np.array(cl, np.int32)
    R = B * S
    kc_ref, _ = oracle.fp4_quant_rows(c["k"])
    ref, _ = oracle.score(c["q"], c["w"], kc_ref, B, S, H, T, c["cl"])
    ids_ref = oracle.select_blocks(ref, c["cl"], ctb, cbs)
    kc = fp4_cache(c["k"])
    sc = t.full((R, T), float("nan"), dtype=t.float32, device="cuda")
    hist = t.full((R, 2048), 3, dtype=t.int32, device="cuda")
    idx.idx_clear_key_hist(hist)
    ids = t.full((R, ids_ref.shape[1]), -7, dtype=t.int32, device="cuda")
    ws = t.empty(idx.idx_select_workspace_size(R, T, ctb, cbs), dtype=t.uint8, device="cuda")
    idx.idx_score_select_blocks(dev(c["q"]), dev(c["w"]), kc, B, S, T, dev(c["cl"]), sc, ctb, cbs,
                                ids, ws, key_hist=hist)
    sync()
    got = host(sc)
    for r in range(R):
        n = max(0, min(int(c["cl"][r]), T))
        assert np.array_equal(bits(got[r, :n]), bits(ref[r, :n])), r
    assert np.array_equal(host(hist).astype(np.int64), _counted_hist(ref, c["cl"], T))
    assert np.array_equal(host(ids), ids_ref)


L2_CASES = [
    # (seed, B, H, T, cbs, ids per row, k, cl override)
    (141, 4, 64, 65536, 128, "select", 2048, None),            # the two-level workload's shape
    (142, 2, 32, 20000, 128, "select", 500, [20000, 9000]),    # 32 heads, cl cuts blocks
    (143, 3, 64, 5000, 64, "messy", 300, None),                # skipped ids in between
    (144, 2, 64, 4096, 128, "few", 2048, None),                # fewer finite candidates than k
    (145, 2, 64, 600, 128, "select", 2048, None),              # k >= T: the closed form
]


@pytest.mark.parametrize("case", L2_CASES)
def test_score_topk_candidates_matches_two_calls(idx, case):
    t = torch()
    seed, B, H, T, cbs, mode, k, cl = case
    say("level two", case)
    c = small_case(seed, B, 1, H, T)
    if cl is not None:
        c["cl"] = np.array(cl, np.int32)
    rng = np.random.default_rng(seed)
    nb = (T + cbs - 1) // cbs
    if mode == "select":
        ids = np.stack([np.sort(rng.choice(nb, size=min(16, nb), replace=False))
                        for _ in range(B)]).astype(np.int32)
    elif mode == "messy":
        # strictly ascending valid ids with skipped ones (negative, past the
        # row's blocks) in between, as idx_topk_candidates takes them
        ids = np.array([[-1, 0, 3, nb + 5, 7, 12, -4, 40],
                        [1, 2, -4, 8, 9, 11, nb + 1, 70],
                        [0, 1, 2, 3, 4, 5, 6, 78]], np.int32)[:B]
    else:
        ids = np.array([[1, 5], [0, 31]], np.int32)[:B]
    kc_ref, _ = oracle.fp4_quant_rows(c["k"])
    ref_ids = np.where((ids >= 0) & (ids < nb), ids, -1)
    ref, _ = oracle.score(c["q"], c["w"], kc_ref, B, 1, H, T, c["cl"], cand=ref_ids, cbs=cbs)
    kc = fp4_cache(c["k"])
    q, w, cld, idd = dev(c["q"]), dev(c["w"]), dev(c["cl"]), dev(ids)
    kout = min(k, T)
    V = ids.shape[1] * cbs
    outs = []
    for fused in (True, False):
        hist = t.zeros((B, 2048), dtype=t.int32, device="cuda")
        out = t.full((B, kout), -9, dtype=t.int32, device="cuda")
        if fused:
            sc = t.full((B, V + 5), float("nan"), dtype=t.float32, device="cuda")
            ko = idx.idx_score_topk_candidates(q, w, kc, B, 1, T, cld, idd, cbs, sc, k, 7, out,
                                               key_hist=hist)
        else:
            sc = t.full((B, T), float("nan"), dtype=t.float32, device="cuda")
            idx.idx_score(q, w, kc, B, 1, T, cld, sc, cand_blocks=idd, cand_block_size=cbs,
                          key_hist=hist)
            ko = idx.idx_topk_candidates(sc, T, cld, idd, cbs, k, 7, out, key_hist=hist)
        sync()
        assert ko == kout
        assert not host(hist).any()  # consumed and reset
        outs.append((host(out), host(sc)))
    (o_f, s_f), (o_2, s_2) = outs
    assert np.array_equal(o_f, o_2)
    assert np.array_equal(o_f, oracle.topk(ref, c["cl"], k, 7))
    # slot scores at their reachable positions equal the oracle's
    for r in range(B):
        for v in range(V):
            blk = ids[r, v // cbs]
            if blk < 0 or blk >= nb:
                continue
            p = blk * cbs + v % cbs
            if p < min(int(c["cl"][r]), T):
                assert bits(s_f[r, v:v + 1])[0] == bits(ref[r, p:p + 1])[0], (r, v, p)
    assert np.all(np.isnan(s_f[:, V:]))  # nothing past the slots


TL_CASES = [
    # (seed, B, H, T, cbs, ids per row, k, cl override): level one split path
    # and level two's 1024-thread ranking side by side, or the two in order
    (151, 4, 64, 65536, 128, 64, 2048, None),                 # side by side: the workload's shape
    (152, 3, 32, 50000, 128, 40, 2048, [50000, 40000, 1]),   # side by side, 32 heads, short rows
    (153, 2, 64, 20000, 128, 24, 500, None),                  # level one on one workgroup: in order
    (154, 2, 64, 65536, 64, 16, 2048, None),                  # level two on 256 threads: in order
]


@pytest.mark.parametrize("case", TL_CASES)
def test_two_level_topk_equals_the_two_calls(idx, case):
    """idx_two_level_topk against idx_topk then idx_score_topk_candidates on
    the same level-one scores and histogram: both index sets bit for bit,
    both histograms reset, and each equal to the oracle's top-k."""
    t = torch()
    seed, B, H, T, cbs, nid, k, cl = case
    say("two-level top-k", case)
    c = small_case(seed, B, 1, H, T)
    if cl is not None:
        c["cl"] = np.array(cl, np.int32)
    rng = np.random.default_rng(seed)
    w2 = rng.permutation(c["w"].reshape(-1)).reshape(c["w"].shape)  # level two's own weights
    nb = (T + cbs - 1) // cbs
    ids = np.stack([np.sort(rng.choice(nb, size=nid, replace=False)) for _ in range(B)]).astype(np.int32)
    kc_ref, _ = oracle.fp4_quant_rows(c["k"])
    ref1, _ = oracle.score(c["q"], c["w"], kc_ref, B, 1, H, T, c["cl"])
    ref2, _ = oracle.score(c["q"], w2, kc_ref, B, 1, H, T, c["cl"], cand=ids, cbs=cbs)
    kc = fp4_cache(c["k"])
    q, w, wd2, cld, idd = dev(c["q"]), dev(c["w"]), dev(w2), dev(c["cl"]), dev(ids)
    kout = min(k, T)
    V = nid * cbs
    res = []
    for together in (True, False):
        sc1 = t.empty((B, T), dtype=t.float32, device="cuda")
        h1 = t.zeros((B, 2048), dtype=t.int32, device="cuda")
        h2 = t.zeros((B, 2048), dtype=t.int32, device="cuda")
        idx.idx_score(q, w, kc, B, 1, T, cld, sc1, key_hist=h1)
        out1 = t.full((B, kout), -9, dtype=t.int32, device="cuda")
        out2 = t.full((B, kout), -9, dtype=t.int32, device="cuda")
        slot = t.full((B, V), float("nan"), dtype=t.float32, device="cuda")
        if together:
            idx.idx_two_level_topk(sc1, h1, out1, None, q, wd2, kc, B, 1, T, cld, idd, cbs, slot,
                                   h2, k, 3, out2)
        else:
            idx.idx_topk(sc1, T, cld, k, 3, out1, key_hist=h1)
            idx.idx_score_topk_candidates(q, wd2, kc, B, 1, T, cld, idd, cbs, slot, k, 3, out2,
                                          key_hist=h2)
        sync()
        assert not host(h1).any() and not host(h2).any()  # both consumed and reset
        res.append((host(out1), host(out2)))
    (a1, a2), (b1, b2) = res
    assert np.array_equal(a1, b1)
    assert np.array_equal(a2, b2)
    assert np.array_equal(a1, oracle.topk(ref1, c["cl"], k, 3))
    assert np.array_equal(a2, oracle.topk(ref2, c["cl"], k, 3))


def test_two_level_topk_rejects_one_shared_histogram(idx):
    t = torch()
    B, T = 2, 65536
    c = small_case(160, B, 1, 64, T)
    kc = fp4_cache(c["k"])
    h = t.zeros((B, 2048), dtype=t.int32, device="cuda")
    sc1 = t.empty((B, T), dtype=t.float32, device="cuda")
    out = t.empty((B, 2048), dtype=t.int32, device="cuda")
    slot = t.empty((B, 8192), dtype=t.float32, device="cuda")
    ids = dev(np.tile(np.arange(64, dtype=np.int32), (B, 1)))
    with pytest.raises(idx.IdxError):
        idx.idx_two_level_topk(sc1, h, out, None, dev(c["q"]), dev(c["w"]), kc, B, 1, T,
                               dev(c["cl"]), ids, 128, slot, h, 2048, 0, out)
