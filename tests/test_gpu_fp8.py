"""GPU parity of the FP8 indexer cache ([VLLM] "attention.py" patch,
_indexer_k_cache_head_dim: 128 e4m3 bytes plus one fp32 ue8m0 scale per 128
values) against the CPU oracle.

Contract (a 128-term e4m3 dot is not exact in fp32, so the matrix core's
summation shows in the last bits):
- quantised rows, round trips and published rows: bit-exact;
- scores: |a - b| <= 2^-14 * sum_h |w_h| * sum_i |q_hi k_ti| (dequantised
  values) against the oracle's scores (exactly rounded dots, the same fixed
  head order).  This bound follows from the arithmetic: relu is 1-Lipschitz,
  so a score moves by at most sum_h |w_h| times its heads' dot errors, and
  each e4m3 dot of the matrix core was measured within 2^-16.4 of its
  sum |q_i k_i| (unbiased; 14% exact); 2^-14 leaves a margin of about 2.6.
  The error against the row's largest score (about 1e-5) and the fraction
  bit-identical are printed;
- indices: bit-exact against the oracle's top-k of the GPU's own scores, and
  a valid top-k of the oracle's scores within the same bound (every selected
  oracle score >= every unselected one minus the bounds of both);
- on fp4 round trips with equal block scales (exactly representable in
  e4m3, so every dot is exact) the FP8 scores equal the oracle's bit for bit.
"""
import numpy as np
import pytest

import oracle
from sparse_attention_top_fp4_amd.inputs import (YARN, bf16_bits, bf16_to_f32, generate,
                                                 head_weights, normal_bf16, small_case, workload)

from gpu_util import bits, dev, host, say, sync, torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def idx():
    import sparse_attention_top_fp4_amd as m
    m.load_library()
    return m


def fp8_cache(idx, k):
    t = torch()
    rows = t.empty(k.shape[:-1] + (132,), dtype=t.uint8, device="cuda")
    idx.idx_fp8_quant(dev(k), rows)
    return rows


DOT_ERR = 2.0 ** -14  # per head, relative to sum |q_i k_i|


def score_bound(q, w, k, S):
    """Per (row, position) bound of the contract: DOT_ERR * sum_h |w_h| *
    sum_i |q_hi k_ti|, from the FP8 round trips of q [R][H][128] and k
    [B][T][128] (float64) and the weights w [R][H]."""
    _, qrt = oracle.fp8_quant_rows(q)
    _, krt = oracle.fp8_quant_rows(k)
    qa = np.abs(bf16_to_f32(qrt).astype(np.float64))
    ka = np.abs(bf16_to_f32(krt).astype(np.float64))
    wa = np.abs(bf16_to_f32(w).astype(np.float64))
    out = np.empty((q.shape[0], k.shape[1]))
    for r in range(q.shape[0]):
        out[r] = DOT_ERR * (wa[r] @ (qa[r] @ ka[r // S].T))
    return out


def close(a, b, bound):
    """-inf must match exactly; finite scores within the bound.  Returns
    (ok, worst error over the bound, worst error over the row's largest
    |score|)."""
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    fin = np.isfinite(b)
    assert np.array_equal(np.isfinite(a), fin)
    err = np.where(fin, np.abs(a - np.where(fin, b, 0.0)), 0.0)
    over = float((err / np.maximum(bound, 1e-300)).max())
    rowmax = np.where(fin, np.abs(b), 0.0).max(axis=-1, keepdims=True)
    rel = float((err / np.maximum(rowmax, 1e-300)).max())
    return bool(np.all(err <= bound)), over, rel


def valid_selection(out, s_ref, cl, kout, offset, bound):
    """out: GPU indices of a row; s_ref: oracle scores.  The kept positions
    must be a top-k of s_ref within the bound."""
    for r in range(out.shape[0]):
        c = int(min(cl[r], s_ref.shape[1]))
        sel = out[r][out[r] >= 0] - offset
        assert len(sel) == min(kout, c)
        mask = np.zeros(s_ref.shape[1], bool)
        mask[sel] = True
        reach = np.arange(s_ref.shape[1]) < c
        if mask[reach].all() or not mask[reach].any():
            continue
        srow = s_ref[r].astype(np.float64)
        b = bound[r]
        lo = (srow + b)[mask].min()
        hi = (srow - b)[reach & ~mask].max()
        assert lo >= hi, f"row {r}"


def test_fp8_quant_every_bf16_at_several_scales(idx):
    t = torch()
    allb = np.arange(0x10000, dtype=np.uint32).astype(np.uint16)
    vals = bf16_to_f32(allb)
    fin = allb[np.isfinite(vals)]
    for anchor in (448.0, 1.0, 3.0e-30, 7.5e20, 0.0):
        say("fp8 quant, block anchor", anchor)
        v = bf16_to_f32(fin)
        if anchor:
            keep = fin[np.abs(v) <= anchor]
        else:
            keep = fin[v == 0]
        n = -(-len(keep) // 127)
        x = np.zeros((n, 128), np.uint16)
        x[:, 0] = bf16_bits(np.float32(anchor))
        flat = np.zeros(n * 127, np.uint16)
        flat[:len(keep)] = keep
        x[:, 1:] = flat.reshape(n, 127)
        rows_ref, rt_ref = oracle.fp8_quant_rows(x)
        rows = t.empty((n, 132), dtype=t.uint8, device="cuda")
        rt = t.empty((n, 128), dtype=t.int16, device="cuda")
        idx.idx_fp8_quant(dev(x), rows, rt)
        sync()
        assert np.array_equal(host(rows), rows_ref)
        assert np.array_equal(host(rt, np.uint16), rt_ref)


SCORE_CASES = [
    # (seed, B, S, H, T, start_pos, cand rows, cbs, k)
    (401, 2, 1, 64, 777, None, None, 0, 100),      # ragged tail, several tiles
    (402, 1, 9, 64, 3000, 9000, None, 0, 2048),    # chunked prefill rows
    (403, 3, 1, 32, 4100, None, None, 0, 2048),    # 32 heads
    (404, 2, 1, 64, 20000, None, [list(range(0, 128, 2)), list(range(1, 128, 2))], 128, 2048),
    (405, 2, 1, 64, 40000, None, None, 0, 2048),   # split top-k rows
]


@pytest.mark.parametrize("case", SCORE_CASES)
def test_fp8_score_and_topk(idx, case):
    t = torch()
    seed, B, S, H, T, sp, cand_rows, cbs, k = case
    say("fp8 score", case[:6], cbs, k)
    c = small_case(seed, B, S, H, T, start_pos=sp)
    R = B * S
    kc_ref, _ = oracle.fp8_quant_rows(c["k"])
    cand = None if cand_rows is None else np.array(cand_rows, np.int32)
    ref, _ = oracle.score_fp8(c["q"], c["w"], kc_ref, B, S, H, T, c["cl"], cand=cand, cbs=cbs)
    kc = fp8_cache(idx, c["k"])
    assert np.array_equal(host(kc), kc_ref)
    sc = t.full((R, T), 7.0, dtype=t.float32, device="cuda")
    hist = t.zeros((R, 2048), dtype=t.int32, device="cuda")
    idx.idx_score_fp8(dev(c["q"]), dev(c["w"]), kc, B, S, T, dev(c["cl"]), sc,
                      cand_blocks=None if cand is None else dev(cand), cand_block_size=cbs,
                      key_hist=hist)
    kout = min(k, T)
    out = t.full((R, kout), -7, dtype=t.int32, device="cuda")
    if cand is None:
        idx.idx_topk(sc, T, dev(c["cl"]), k, 3, out, key_hist=hist)
    else:
        idx.idx_topk_candidates(sc, T, dev(c["cl"]), dev(cand), cbs, k, 3, out, key_hist=hist)
    sync()
    got = host(sc)
    tt = np.arange(T)[None, :]
    reach = tt < np.minimum(c["cl"], T)[:, None]
    if cand is not None:
        got = np.where(reach, got, -np.inf)  # -inf outside the candidates, beyond cl unspecified
    else:
        got = np.where(reach, got, -np.inf)
        ref = np.where(reach, ref, -np.inf)
    bound = score_bound(c["q"], c["w"], c["k"], S)
    ok, over, rel = close(got, ref, bound)
    same = float(np.mean(bits(got[np.isfinite(ref)]) == bits(ref[np.isfinite(ref)])))
    say("fp8 score: worst error / bound", over, "worst error / row max", rel,
        "bit-identical fraction", same)
    assert ok
    gi = host(out)
    assert np.array_equal(gi, oracle.topk(got, c["cl"], k, 3))
    valid_selection(gi, ref, c["cl"], kout, 3, bound)
    assert not host(hist).any()


def test_fp8_score_exact_on_shared_grid(idx):
    """fp4 round trips with equal block scales are exact in e4m3: every fp8
    dot is then exact and the GPU scores equal the oracle's bit for bit (and
    the fp4 path's)."""
    t = torch()
    rng = np.random.default_rng(17)
    B, S, H, T = 2, 1, 64, 1000

    def grid(x):
        x = bf16_to_f32(x).copy()
        x[..., ::32] = 5.5
        _, rt = oracle.fp4_quant_rows(bf16_bits(x))
        return rt

    q = grid(normal_bf16(rng, (B * S, H, 128)))
    k = grid(normal_bf16(rng, (B, T, 128)))
    w = head_weights(rng, B * S, H)
    cl = np.array([T, 613], np.int32)
    kc8, _ = oracle.fp8_quant_rows(k)
    ref, _ = oracle.score_fp8(q, w, kc8, B, S, H, T, cl)
    sc = t.empty((B * S, T), dtype=t.float32, device="cuda")
    idx.idx_score_fp8(dev(q), dev(w), fp8_cache(idx, k), B, S, T, dev(cl), sc)
    sync()
    got = host(sc)
    for r in range(B * S):
        n = int(cl[r])
        assert np.array_equal(bits(got[r, :n]), bits(ref[r, :n])), f"row {r}"


def test_fp8_publish(idx):
    t = torch()
    say("fp8 publish")
    rng = np.random.default_rng(23)
    B, tcap = 4, 300
    start_pos = 4 * 250 - 1
    latent = normal_bf16(rng, (B, 1, 512))
    wk = normal_bf16(rng, (128, 512), std=0.02)
    gamma = np.ones(128, np.float32)
    cs = oracle.yarn_cos_sin(1200, 64, YARN["theta"], YARN["factor"], YARN["orig_len"],
                             YARN["beta_fast"], YARN["beta_slow"])
    kc4 = np.zeros((B, tcap, 68), np.uint8)
    pre = oracle.publish(latent, wk, gamma, cs, start_pos, 4, 1e-6, kc4)
    row_ref, _ = oracle.fp8_quant_rows(pre[:, 0])
    kc0 = rng.integers(0, 256, size=(B, tcap, 132), dtype=np.uint8)
    kc = dev(kc0)
    idx.idx_publish_keys_fp8(dev(latent), dev(wk), dev(gamma), dev(cs), start_pos, 4, 1e-6, kc)
    sync()
    got = host(kc)
    row = start_pos // 4
    assert np.array_equal(got[:, row], row_ref)
    others = np.ones(tcap, bool)
    others[row] = False
    assert np.array_equal(got[:, others], kc0[:, others])


def test_fp8_batched_decode_128k(idx):
    """The batched decode workload (64 x 32768 keys) on the FP8 cache, as
    `bench.py --fp8` runs it: every row's indices against the oracle's top-k
    of the GPU scores, sampled rows' scores and selections against the
    oracle."""
    from sparse_attention_top_fp4_amd.pipeline import IndexerStep
    wl = workload(1)
    say("fp8 workload", wl.name)
    inp = generate(wl)
    st = IndexerStep(wl, inp, fp8=True)
    st.step()
    sync()
    scores, out = host(st.scores), host(st.out)
    assert np.array_equal(out, oracle.topk(scores, inp["cl"], wl.topk, wl.offset))
    for r in (0, 41):
        kc, _ = oracle.fp8_quant_rows(inp["k"][r])
        assert np.array_equal(host(st.k_cache[r]), kc)
        ref, _ = oracle.score_fp8(inp["q"][r:r + 1], inp["w"][r:r + 1], kc[None], 1, 1, wl.H,
                                  wl.T, inp["cl"][r:r + 1])
        bound = score_bound(inp["q"][r:r + 1], inp["w"][r:r + 1], inp["k"][r:r + 1], 1)
        ok, over, rel = close(scores[r:r + 1], ref, bound)
        say("fp8 workload row", r, "worst error / bound", over, "worst error / row max", rel)
        assert ok
        valid_selection(out[r:r + 1], ref, inp["cl"][r:r + 1], st.kout, wl.offset, bound)
