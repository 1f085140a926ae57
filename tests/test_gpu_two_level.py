"""GPU parity of idx_score_select_blocks, the level-one pass of the
two-level indexer: the scores (bit-identical to the oracle's below
compress_lens), the score histogram (exact counts of the scored positions)
and the selected block ids (bit-exact against the oracle's block select on
its own scores).  Cases take the single-launch form (block maxima from the
score launch, one wave per row ranks them) and both two-call forms (blocks
that straddle score chunks; more blocks than one wave ranks), with rows whose
compress_lens is T, a part of T, 1 and 0, decode and prefill rows, and 32
and 64 heads."""
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
