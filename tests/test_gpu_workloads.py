"""The five synthetic workloads at full size, run through the same pipeline
and launch configuration the benchmark times, checked against the CPU
oracle: sampled rows element by element (key cache bytes, every score of the
row, the row's indices), every row's indices against the oracle's top-k of
the GPU scores (all 32768 rows of the prefill included), and the output
invariants on every row.

Workloads (seeded; no dataset): tiny decode (1 x 512 keys), batched decode
at 128K tokens (64 x 32768), causal prefill (32768 queries over 8192 keys),
two-level selection (16 x 65536, 64 blocks of 128), long decode with a key
publish (4 x 262144)."""
import numpy as np
import pytest

import oracle
from sparse_attention_top_fp4_amd.inputs import YARN, generate, workload

from gpu_util import bits, host, say, sync, torch

pytestmark = pytest.mark.gpu


def _run(cid):
    """One step with the scores kept; where the step is a single fused
    launch, also the step the benchmark times (scores not written), whose
    indices must be the same."""
    from sparse_attention_top_fp4_amd.pipeline import IndexerStep
    wl = workload(cid)
    say("workload", cid, wl.name, "generating")
    inp = generate(wl)
    say("workload", cid, "step")
    st = IndexerStep(wl, inp)
    st.step()
    if st.fused:
        lean = IndexerStep(wl, inp, keep_scores=False)
        lean.step()
        sync()
        assert lean.scores is None
        assert np.array_equal(host(lean.out), host(st.out))
    sync()
    return wl, inp, st


def _invariants(out, cl, kout, offset):
    """Width, -1 count and placement, position order, range, on every row."""
    R = out.shape[0]
    assert out.shape == (R, kout)
    neg = out == -1
    n_neg = neg.sum(axis=1)
    assert np.array_equal(n_neg, np.maximum(0, kout - cl.astype(np.int64)))
    valid_cols = kout - n_neg
    col = np.arange(kout)[None, :]
    assert np.array_equal(neg, col >= valid_cols[:, None])  # -1 only at the tail
    v = np.where(neg, np.iinfo(np.int32).max, out.astype(np.int64))
    d = np.diff(v, axis=1)
    assert np.all((d > 0) | (np.isin(d, [0]) & neg[:, 1:]))  # strictly ascending valid part
    vv = out[~neg] - offset
    assert np.all(vv >= 0)


def _sampled_rows_vs_oracle(wl, inp, st, rows, scores_gpu, out_gpu, w_key="w", cand=None,
                            kc_full=None):
    kc = kc_full
    for r in rows:
        b = r // wl.S
        if kc_full is None:
            kc, _ = oracle.fp4_quant_rows(inp["k"][b])
            kc = kc[None]
            assert np.array_equal(host(st.k_cache[b]), kc[0]), "key cache bytes differ"
            kb = kc
        else:
            kb = kc_full[b:b + 1]
        cl = inp["cl"][r:r + 1]
        ref, inexact = oracle.score(inp["q"][r:r + 1], inp[w_key][r:r + 1], kb, 1, 1, wl.H, wl.T,
                                    cl, cand=None if cand is None else cand[r:r + 1],
                                    cbs=wl.cbs)
        assert inexact == 0
        n = int(min(cl[0], wl.T)) if cand is None else wl.T
        got = scores_gpu[r] if scores_gpu.ndim == 2 else scores_gpu
        assert np.array_equal(bits(got[:n]), bits(ref[0, :n])), f"row {r} scores"
        ref_idx = oracle.topk(ref, cl, wl.topk, wl.offset)
        assert np.array_equal(out_gpu[r], ref_idx[0]), f"row {r} indices"


def test_tiny_decode_full():
    wl, inp, st = _run(0)
    kc, _ = oracle.fp4_quant_rows(inp["k"])
    assert np.array_equal(host(st.k_cache), kc)
    ref, inexact = oracle.score(inp["q"], inp["w"], kc, wl.B, wl.S, wl.H, wl.T, inp["cl"])
    assert inexact == 0
    assert np.array_equal(bits(host(st.scores)), bits(ref))
    assert np.array_equal(host(st.out), oracle.topk(ref, inp["cl"], wl.topk, wl.offset))


def test_batched_decode_128k():
    wl, inp, st = _run(1)
    scores, out = host(st.scores), host(st.out)
    _invariants(out, inp["cl"], st.kout, wl.offset)
    assert np.array_equal(out, oracle.topk(scores, inp["cl"], wl.topk, wl.offset))
    _sampled_rows_vs_oracle(wl, inp, st, [0, 37, 63], scores, out)


def test_causal_prefill_32k():
    wl, inp, st = _run(2)
    out = host(st.out)
    cl = inp["cl"]
    _invariants(out, cl, st.kout, wl.offset)
    kc, _ = oracle.fp4_quant_rows(inp["k"][0])
    assert np.array_equal(host(st.k_cache[0]), kc)
    # every row's indices (those of the launch the benchmark times, which
    # equal the scored launch's) against the oracle's top-k of the GPU
    # scores, 4096 rows at a time
    for r0 in range(0, wl.R, 4096):
        say("workload", 2, "rows", r0, "against the oracle's top-k")
        sc_chunk = host(st.scores[r0:r0 + 4096])
        ref_idx = oracle.topk(sc_chunk, cl[r0:r0 + 4096], wl.topk, wl.offset)
        bad = np.nonzero((out[r0:r0 + 4096] != ref_idx).any(axis=1))[0]
        assert bad.size == 0, f"rows {(bad[:8] + r0).tolist()} differ"
        del sc_chunk
    rows = np.array([0, 3, 4, 7, 8, 1000, 8191, 8192, 8195, 16383, 20000, 32767])
    sc_rows = host(st.scores[torch().as_tensor(rows, device="cuda")])
    # scores and indices of the sampled rows against the oracle end to end
    ref, inexact = oracle.score(inp["q"][rows], inp["w"][rows], kc[None], 1, len(rows), wl.H,
                                wl.T, cl[rows])
    assert inexact == 0
    for i, r in enumerate(rows):
        n = int(cl[r])
        assert np.array_equal(bits(sc_rows[i, :n]), bits(ref[i, :n])), f"row {r}"
    assert np.array_equal(out[rows], oracle.topk(ref, cl[rows], wl.topk, wl.offset))


def test_two_level_256k():
    wl, inp, st = _run(3)
    s1, ids, o1 = host(st.scores), host(st.ids), host(st.out_l1)
    s2, out = host(st.level_two_rows()), host(st.out)
    cl = inp["cl"]
    _invariants(out, cl, st.kout, wl.offset)
    _invariants(o1, cl, st.kout, wl.offset)
    # every row: selection and both top-k against the oracle applied to GPU scores
    assert np.array_equal(ids, oracle.select_blocks(s1, cl, wl.ctb, wl.cbs))
    assert np.array_equal(o1, oracle.topk(s1, cl, wl.topk, wl.offset))
    assert np.array_equal(out, oracle.topk(s2, cl, wl.topk, wl.offset))
    for r in (0, 9):
        kc, _ = oracle.fp4_quant_rows(inp["k"][r])
        assert np.array_equal(host(st.k_cache[r]), kc)
        ref1, _ = oracle.score(inp["q"][r:r + 1], inp["w"][r:r + 1], kc[None], 1, 1, wl.H, wl.T,
                               cl[r:r + 1])
        assert np.array_equal(bits(s1[r]), bits(ref1[0])), f"row {r} level one"
        rid = oracle.select_blocks(ref1, cl[r:r + 1], wl.ctb, wl.cbs)
        assert np.array_equal(ids[r], rid[0])
        ref2, _ = oracle.score(inp["q"][r:r + 1], inp["w2"][r:r + 1], kc[None], 1, 1, wl.H, wl.T,
                               cl[r:r + 1], cand=rid, cbs=wl.cbs)
        assert np.array_equal(bits(s2[r]), bits(ref2[0])), f"row {r} level two"
        assert np.array_equal(out[r], oracle.topk(ref2, cl[r:r + 1], wl.topk, wl.offset)[0])
    # two more steps back to back, as the benchmark issues them: the score
    # histogram must be back at zero before each step's score refills it
    say("workload", 3, "two more steps")
    st.step()
    st.step()
    sync()
    assert np.array_equal(host(st.out_l1), o1)
    assert np.array_equal(host(st.out), out)
    assert np.array_equal(host(st.ids), ids)


def test_long_decode_publish_1m():
    from sparse_attention_top_fp4_amd.inputs import YARN
    wl, inp, st = _run(4)
    assert st.publish_in_score  # the new key is published inside the score launch
    scores, out = host(st.scores), host(st.out)
    cl = inp["cl"]
    _invariants(out, cl, st.kout, wl.offset)
    assert np.array_equal(out, oracle.topk(scores, cl, wl.topk, wl.offset))
    pos = wl.start_pos + 1 - wl.ratio
    row = wl.start_pos // wl.ratio
    cs = oracle.yarn_cos_sin(pos + 1, wl.rd, YARN["theta"], YARN["factor"], YARN["orig_len"],
                             YARN["beta_fast"], YARN["beta_slow"])
    for b in (1, 3):
        kc, _ = oracle.fp4_quant_rows(inp["k"][b])
        kc = kc[None].copy()
        oracle.publish(inp["latent"][b:b + 1], inp["wk"], inp["gamma"], cs, wl.start_pos,
                       wl.ratio, wl.eps, kc)
        got = host(st.k_cache[b])
        assert np.array_equal(got[row], kc[0, row]), "published key row"
        assert np.array_equal(got, kc[0])
        ref, inexact = oracle.score(inp["q"][b:b + 1], inp["w"][b:b + 1], kc, 1, 1, wl.H, wl.T,
                                    cl[b:b + 1])
        assert inexact == 0
        assert np.array_equal(bits(scores[b]), bits(ref[0])), f"row {b}"
        assert np.array_equal(out[b], oracle.topk(ref, cl[b:b + 1], wl.topk, wl.offset)[0])


def test_causal_prefill_with_prompt_publish():
    """The prefill step publishing its 8192 prompt keys first (key publish of
    many groups at positions 4j), then scoring them: every cache row against
    the oracle's publish, and sampled rows' scores and indices."""
    from sparse_attention_top_fp4_amd.inputs import publish_inputs
    from sparse_attention_top_fp4_amd.pipeline import IndexerStep
    wl = workload(2)
    say("workload", 2, "prompt publish: generating")
    inp = generate(wl)
    G = wl.S // wl.ratio
    inp.update(publish_inputs(wl, G, wl.seed() + 1000))
    st = IndexerStep(wl, inp, publish=True)
    say("workload", 2, "prompt publish: step")
    st.step()
    sync()
    cs = oracle.yarn_cos_sin(G * wl.ratio, wl.rd, YARN["theta"], YARN["factor"],
                             YARN["orig_len"], YARN["beta_fast"], YARN["beta_slow"])
    kc = np.zeros((1, wl.T, 68), np.uint8)
    oracle.publish(inp["latent"], inp["wk"], inp["gamma"], cs, 0, wl.ratio, wl.eps, kc)
    assert np.array_equal(host(st.k_cache), kc)
    cl = inp["cl"]
    rows = np.array([8191, 8192, 20000, 32767])
    ref, _ = oracle.score(inp["q"][rows], inp["w"][rows], kc, 1, len(rows), wl.H, wl.T, cl[rows])
    sc = host(st.scores[torch().as_tensor(rows, device="cuda")])
    for i, r in enumerate(rows):
        n = int(cl[r])
        assert np.array_equal(bits(sc[i, :n]), bits(ref[i, :n])), f"row {r}"
    assert np.array_equal(host(st.out)[rows], oracle.topk(ref, cl[rows], wl.topk, wl.offset))
