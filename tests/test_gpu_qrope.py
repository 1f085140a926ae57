"""GPU parity of the query step (RoPE on the query heads' last rd dims at
positions start_pos + s, fp4 quantise, weight scaling) against the oracle:
quantised rows, their round trip and the scaled weights bit-exact; and the
round trip, given to the score as q, gives the scores of the rows."""
import numpy as np
import pytest

import oracle
from sparse_attention_top_fp4_amd.inputs import YARN, normal_bf16

from gpu_util import bits, dev, fp4_cache, host, say, sync, torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def idx():
    import sparse_attention_top_fp4_amd as m
    m.load_library()
    return m


@pytest.mark.parametrize("B,S,H,sp,rd", [(4, 1, 64, 131071, 64), (1, 40, 64, 0, 64),
                                         (2, 7, 32, 1000, 40), (3, 2, 64, 5, 0),
                                         (1, 3, 32, 7, 64),    # 96 heads: a partial workgroup
                                         (2, 5, 64, 300, 42),  # RoPE from dim 86, inside a piece
                                         (1, 1, 1, 3, 2),      # one head, one RoPE pair
                                         (1, 2, 16, 9, 128)])  # every dim rotated
def test_q_rope_quant_matches_oracle(idx, B, S, H, sp, rd):
    t = torch()
    say("q rope quant", B, S, H, sp, rd)
    rng = np.random.default_rng(B * 100 + S)
    R = B * S
    q = normal_bf16(rng, (R, H, 128))
    w = normal_bf16(rng, (R, H))
    scale = np.float32(128 ** -0.5 * H ** -0.5)
    P = sp + S
    cs = (oracle.yarn_cos_sin(P, rd, YARN["theta"], YARN["factor"], YARN["orig_len"],
                              YARN["beta_fast"], YARN["beta_slow"]) if rd
          else np.zeros((P, 0, 2), np.float32))
    rows_ref, rt_ref, _, w_ref = oracle.q_rope_quant(q, w, scale, cs, sp, S, rd=rd)
    rows = t.full((R, H, 68), 7, dtype=t.uint8, device="cuda")
    rt = t.zeros((R, H, 128), dtype=t.int16, device="cuda")
    w_out = t.zeros((R, H), dtype=t.int16, device="cuda")
    csd = dev(cs) if rd else t.zeros((P, 1, 2), dtype=t.float32, device="cuda")
    idx.idx_q_rope_quant(dev(q), dev(w), float(scale), csd, sp, S, rows, w_out, q_roundtrip=rt,
                         rd=rd)
    sync()
    assert np.array_equal(host(rows), rows_ref)
    assert np.array_equal(host(rt, np.uint16), rt_ref)
    assert np.array_equal(host(w_out, np.uint16), w_ref)


def test_round_trip_is_a_valid_score_query(idx):
    """The step's outputs feed idx_score: its scores equal the oracle's score
    of the rotated, quantised heads with the scaled weights."""
    t = torch()
    say("q rope quant -> score")
    rng = np.random.default_rng(5)
    B, S, H, T, sp = 2, 3, 64, 700, 2797
    R = B * S
    q = normal_bf16(rng, (R, H, 128))
    w = normal_bf16(rng, (R, H))
    k = normal_bf16(rng, (B, T, 128))
    scale = np.float32(128 ** -0.5 * H ** -0.5)
    cs = oracle.yarn_cos_sin(sp + S, 64, YARN["theta"], YARN["factor"], YARN["orig_len"],
                             YARN["beta_fast"], YARN["beta_slow"])
    _, rt_ref, _, w_ref = oracle.q_rope_quant(q, w, scale, cs, sp, S)
    cl = np.array([(sp + s + 1) // 4 for _ in range(B) for s in range(S)], np.int32)
    kc_ref, _ = oracle.fp4_quant_rows(k)
    ref, _ = oracle.score(rt_ref, w_ref, kc_ref, B, S, H, T, cl)
    rows = t.empty((R, H, 68), dtype=t.uint8, device="cuda")
    rt = t.empty((R, H, 128), dtype=t.int16, device="cuda")
    w_out = t.empty((R, H), dtype=t.int16, device="cuda")
    idx.idx_q_rope_quant(dev(q), dev(w), float(scale), dev(cs), sp, S, rows, w_out, q_roundtrip=rt)
    sc = t.full((R, T), float("nan"), dtype=t.float32, device="cuda")
    idx.idx_score(rt, w_out, fp4_cache(k), B, S, T, dev(cl), sc)
    sync()
    g = host(sc)
    for r in range(R):
        assert np.array_equal(bits(g[r, :cl[r]]), bits(ref[r, :cl[r]])), r


@pytest.mark.parametrize("fused,H", [(False, 64), (True, 64), (False, 32), (True, 32)])
def test_score_takes_the_quantised_rows(idx, fused, H):
    """idx_score_q4 / idx_score_topk_q4 on the query step's rows give the
    scores and indices of the oracle (and of idx_score on the round trip)."""
    t = torch()
    say("score from quantised rows", fused, H)
    rng = np.random.default_rng(8 + H)
    B, S, T, sp = 2, 6, 3000, 10000
    R = B * S
    q = normal_bf16(rng, (R, H, 128))
    w = normal_bf16(rng, (R, H))
    k = normal_bf16(rng, (B, T, 128))
    cs = oracle.yarn_cos_sin(sp + S, 64, YARN["theta"], YARN["factor"], YARN["orig_len"],
                             YARN["beta_fast"], YARN["beta_slow"])
    _, rt_ref, _, w_ref = oracle.q_rope_quant(q, w, 1.0, cs, sp, S)
    cl = np.array([(sp + s + 1) // 4 for _ in range(B) for s in range(S)], np.int32)
    cl = np.minimum(cl, T)
    kc_ref, _ = oracle.fp4_quant_rows(k)
    ref, _ = oracle.score(rt_ref, w_ref, kc_ref, B, S, H, T, cl)
    rows = t.empty((R, H, 68), dtype=t.uint8, device="cuda")
    rt = t.empty((R, H, 128), dtype=t.int16, device="cuda")
    w_out = t.empty((R, H), dtype=t.int16, device="cuda")
    idx.idx_q_rope_quant(dev(q), dev(w), 1.0, dev(cs), sp, S, rows, w_out, q_roundtrip=rt)
    kc = fp4_cache(k)
    sc = t.full((R, T), float("nan"), dtype=t.float32, device="cuda")
    sc2 = t.full((R, T), float("nan"), dtype=t.float32, device="cuda")
    if fused:
        k_top = 700
        out = t.full((R, k_top), -7, dtype=t.int32, device="cuda")
        idx.idx_score_topk_q4(rows, w_out, kc, B, S, T, dev(cl), k_top, 2, out, scores=sc)
        idx.idx_score_topk(rt, w_out, kc, B, S, T, dev(cl), k_top, 2,
                           t.empty_like(out), scores=sc2)
        sync()
        assert np.array_equal(host(out), oracle.topk(ref, cl, k_top, 2))
    else:
        hist = t.zeros((R, 2048), dtype=t.int32, device="cuda")
        hist2 = t.zeros((R, 2048), dtype=t.int32, device="cuda")
        cand = np.array([[1, 5, 9, 30]] * R, np.int32)  # and the candidate mode
        idx.idx_score_q4(rows, w_out, kc, B, S, T, dev(cl), sc, key_hist=hist)
        idx.idx_score(rt, w_out, kc, B, S, T, dev(cl), sc2, key_hist=hist2)
        sc3 = t.full((R, T), float("nan"), dtype=t.float32, device="cuda")
        idx.idx_score_q4(rows, w_out, kc, B, S, T, dev(cl), sc3, cand_blocks=dev(cand),
                         cand_block_size=64)
        sync()
        assert np.array_equal(host(hist), host(hist2))
        ref_c, _ = oracle.score(rt_ref, w_ref, kc_ref, B, S, H, T, cl, cand=cand, cbs=64)
        assert np.array_equal(bits(host(sc3)), bits(ref_c))
    g, g2 = host(sc), host(sc2)
    for r in range(R):
        n = int(cl[r])
        assert np.array_equal(bits(g[r, :n]), bits(ref[r, :n])), r
        assert np.array_equal(bits(g[r, :n]), bits(g2[r, :n])), r


QS_CASES = [
    # (fused, B, S, H, T, start_pos, rd, w_scale, k)
    (False, 2, 6, 64, 3000, 10000, 64, 1.0, 0),          # decode-like rows, several chunks
    (False, 64, 1, 64, 32768, 131071, 64, 1.0, 0),       # the batched decode's rows (sampled)
    (True, 2, 6, 64, 3000, 10000, 64, 1.0, 700),         # fused top-k
    (True, 1, 9, 32, 5000, 15990, 40, 0.0625, 300),      # 32 heads, rd 40, scaled weights
    (False, 3, 2, 64, 700, 5, 0, 0.5, 0),                # rd 0: no rotation, weights scaled
    (False, 2, 3, 64, 900, 50, 42, 0.25, 0),             # RoPE from dim 86, inside a block
]


@pytest.mark.parametrize("case", QS_CASES)
def test_score_with_query_step_equals_the_two_calls(idx, case):
    """idx_score_qrope / idx_score_topk_qrope: the query step inside the
    score launch gives bit for bit the scores, histogram and indices of
    idx_q_rope_quant then idx_score_q4 / idx_score_topk_q4, and the
    oracle's (checked on up to eight rows)."""
    t = torch()
    fused, B, S, H, T, sp, rd, wsc, k = case
    say("score with the query step", case)
    rng = np.random.default_rng(300 + B * S + H)
    R = B * S
    q = normal_bf16(rng, (R, H, 128))
    w = normal_bf16(rng, (R, H))
    kk = normal_bf16(rng, (B, T, 128))
    P = sp + S
    cs = (oracle.yarn_cos_sin(P, rd, YARN["theta"], YARN["factor"], YARN["orig_len"],
                              YARN["beta_fast"], YARN["beta_slow"]) if rd
          else np.zeros((P, 1, 2), np.float32))
    cl = np.minimum(np.array([(sp + s + 1) // 4 for _ in range(B) for s in range(S)], np.int32), T)
    kc = fp4_cache(kk)
    qd, wd, csd, cld = dev(q), dev(w), dev(cs), dev(cl)
    rows = t.empty((R, H, 68), dtype=t.uint8, device="cuda")
    w_out = t.empty((R, H), dtype=t.int16, device="cuda")
    idx.idx_q_rope_quant(qd, wd, wsc, csd, sp, S, rows, w_out, rd=rd)
    sc1 = t.full((R, T), float("nan"), dtype=t.float32, device="cuda")
    sc2 = t.full((R, T), float("nan"), dtype=t.float32, device="cuda")
    if fused:
        o1 = t.full((R, k), -7, dtype=t.int32, device="cuda")
        o2 = t.full((R, k), -7, dtype=t.int32, device="cuda")
        idx.idx_score_topk_qrope(qd, wd, wsc, csd, sp, kc, B, S, T, cld, k, 2, o1, scores=sc1,
                                 rd=rd)
        idx.idx_score_topk_q4(rows, w_out, kc, B, S, T, cld, k, 2, o2, scores=sc2)
        sync()
        assert np.array_equal(host(o1), host(o2))
    else:
        h1 = t.zeros((R, 2048), dtype=t.int32, device="cuda")
        h2 = t.zeros((R, 2048), dtype=t.int32, device="cuda")
        idx.idx_score_qrope(qd, wd, wsc, csd, sp, kc, B, S, T, cld, sc1, key_hist=h1, rd=rd)
        idx.idx_score_q4(rows, w_out, kc, B, S, T, cld, sc2, key_hist=h2)
        sync()
        assert np.array_equal(host(h1), host(h2))
    g1, g2 = host(sc1), host(sc2)
    assert np.array_equal(bits(np.nan_to_num(g1, nan=7.0)), bits(np.nan_to_num(g2, nan=7.0)))
    # the oracle on a sample of rows
    rs = np.unique(np.linspace(0, R - 1, min(R, 8)).astype(int))
    bsel = sorted({int(r) // S for r in rs})
    _, rt_ref, _, w_ref = oracle.q_rope_quant(q, w, np.float32(wsc), cs, sp, S, rd=rd)
    kc_ref, _ = oracle.fp4_quant_rows(kk[bsel])
    for r in rs:
        b, s = divmod(int(r), S)
        ref, _ = oracle.score(rt_ref[r:r + 1], w_ref[r:r + 1], kc_ref[bsel.index(b):bsel.index(b) + 1],
                              1, 1, H, T, cl[r:r + 1])
        n = int(cl[r])
        assert np.array_equal(bits(g1[r, :n]), bits(ref[0, :n])), r
        if fused:
            assert np.array_equal(host(o1)[r], oracle.topk(ref, cl[r:r + 1], k, 2)[0]), r


def test_bf16_conversion_instruction_matches_rne(idx):
    """The score launch's query step rounds with the gfx950 instruction that
    converts two fp32 values to bf16; the other kernels (and the query
    step's own launch) round in software.  They agree on every finite fp32
    input."""
    say("bf16 conversion instruction, exhaustive")
    assert idx.idx_probe_bf16_convert() == 0
