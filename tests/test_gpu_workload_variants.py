"""The benchmark's two step variants at the full workload sizes, in the
launch configuration it times with them:

- the paged key cache (pages of 64 compressed positions in a seeded random
  order, [VLLM, DeepseekV4IndexerCache]): every output of the step
  bit-identical to the contiguous step's (indices, kept scores below
  compress_lens, level-one candidate ids and indices, the published row),
  with the contiguous step itself checked against the oracle in the
  workload tests; sampled rows also against the oracle directly;
- the query step ([IDX, forward: the query heads' RoPE at start_pos + s,
  fp4_act_quant, weight scaling]): the workload's q taken as the heads
  before RoPE; sampled rows end to end against the oracle's query step and
  score, every row's indices against the oracle's top-k of the GPU scores.
"""
import numpy as np
import pytest

import oracle
from sparse_attention_top_fp4_amd.inputs import YARN, generate, workload

from gpu_util import bits, host, say, sync, torch

pytestmark = pytest.mark.gpu


def _step(wl, inp, **kw):
    from sparse_attention_top_fp4_amd.pipeline import IndexerStep
    st = IndexerStep(wl, inp, **kw)
    st.step()
    return st


def _equal_below_cl(a, b, cl):
    """Bit equality of two device score buffers [R, T] on t < cl[r] (the
    entries past compress_lens are unspecified)."""
    t = torch()
    T = a.shape[1]
    mask = t.arange(T, device="cuda")[None, :] < t.as_tensor(cl, device="cuda")[:, None]
    diff = (a.view(t.int32) != b.view(t.int32)) & mask
    return not bool(diff.any().item())


def _page_rows(st, b, T):
    """Sequence b's rows [T, 68] gathered from a paged step's pool."""
    pool = host(st.k_cache).reshape(st.k_cache.shape[0], -1, 68)
    table = host(st.block_table)
    rows = np.concatenate([pool[table[b, j]] for j in range(table.shape[1])])
    return rows[:T]


@pytest.mark.parametrize("cid", [1, 2, 3, 4])
def test_paged_step_equals_contiguous(cid):
    wl = workload(cid)
    say("paged workload", cid, wl.name, "generating")
    inp = generate(wl)
    cl = inp["cl"]
    say("paged workload", cid, "contiguous step")
    a = _step(wl, inp)
    say("paged workload", cid, "paged step")
    b = _step(wl, inp, paged=True)
    sync()
    assert np.array_equal(host(b.out), host(a.out))
    assert _equal_below_cl(b.scores, a.scores, cl)
    if b.fused:  # the launch the benchmark times: scores not written
        say("paged workload", cid, "paged step, scores not kept")
        lean = _step(wl, inp, paged=True, keep_scores=False)
        sync()
        assert np.array_equal(host(lean.out), host(a.out))
    if b.two_level:
        assert np.array_equal(host(b.ids), host(a.ids))
        assert np.array_equal(host(b.out_l1), host(a.out_l1))
        assert _equal_below_cl(b.level_two_rows(), a.level_two_rows(), cl)
    # a sampled row against the oracle directly, and (publish) the cache
    r = wl.R - 1
    sb = r // wl.S
    kc_seq = _page_rows(b, sb, wl.T)
    assert np.array_equal(kc_seq, host(a.k_cache[sb]))
    if not wl.publish:
        kref, _ = oracle.fp4_quant_rows(inp["k"][sb])
        assert np.array_equal(kc_seq, kref)
    ref, inexact = oracle.score(inp["q"][r:r + 1], inp["w"][r:r + 1], kc_seq[None], 1, 1, wl.H,
                                wl.T, cl[r:r + 1])
    assert inexact == 0
    n = int(cl[r])
    got = host(b.scores[r])
    assert np.array_equal(bits(got[:n]), bits(ref[0, :n]))
    if not b.two_level:
        assert np.array_equal(host(b.out[r]), oracle.topk(ref, cl[r:r + 1], wl.topk,
                                                          wl.offset)[0])


def _oracle_query_rows(wl, inp, rows, cs):
    """The oracle's query step for the given rows (row r at position
    start_pos + r % S): round-trip heads and scaled weights."""
    qs, ws = [], []
    for r in rows:
        _, rt, _, wq = oracle.q_rope_quant(inp["q"][r:r + 1], inp["w"][r:r + 1], 1.0, cs,
                                           wl.start_pos + r % wl.S, 1, rd=wl.rd)
        qs.append(rt[0])
        ws.append(wq[0])
    return np.stack(qs), np.stack(ws)


@pytest.mark.parametrize("cid", [1, 2, 3])
def test_query_step_full(cid):
    wl = workload(cid)
    say("query-step workload", cid, wl.name, "generating")
    inp = generate(wl)
    cl = inp["cl"]
    say("query-step workload", cid, "step")
    st = _step(wl, inp, q_step=True)
    sync()
    out = host(st.out)
    rows = {1: [0, 29, 63], 2: [0, 4, 8191, 20000, 32767], 3: [5, 15]}[cid]
    rows = np.array(rows)
    cs = oracle.yarn_cos_sin(wl.start_pos + wl.S, wl.rd, YARN["theta"], YARN["factor"],
                             YARN["orig_len"], YARN["beta_fast"], YARN["beta_slow"])
    qr, wr = _oracle_query_rows(wl, inp, rows, cs)
    if not st.qrope:  # the query step's own launch leaves its scaled weights
        assert np.array_equal(host(st.w_q, np.uint16)[rows], wr)
    bseq = sorted(set(int(r) // wl.S for r in rows))
    kc = {b: oracle.fp4_quant_rows(inp["k"][b])[0] for b in bseq}
    sc_rows = host(st.scores[torch().as_tensor(rows, device="cuda")])
    for i, r in enumerate(rows):
        b = int(r) // wl.S
        ref, inexact = oracle.score(qr[i:i + 1], wr[i:i + 1], kc[b][None], 1, 1, wl.H, wl.T,
                                    cl[r:r + 1])
        assert inexact == 0
        n = int(cl[r])
        assert np.array_equal(bits(sc_rows[i, :n]), bits(ref[0, :n])), f"row {r}"
        if not st.two_level:
            assert np.array_equal(out[r], oracle.topk(ref, cl[r:r + 1], wl.topk, wl.offset)[0])
    if st.two_level:
        # level one (the candidate source) is a plain top-k of the scores
        assert np.array_equal(host(st.out_l1)[rows],
                              oracle.topk(sc_rows, cl[rows], wl.topk, wl.offset))
    elif cid == 2:
        rng = np.random.default_rng(1)
        extra = rng.choice(wl.R, 256, replace=False)
        sc = host(st.scores[torch().as_tensor(extra, device="cuda")])
        assert np.array_equal(out[extra], oracle.topk(sc, cl[extra], wl.topk, wl.offset))
    else:
        assert np.array_equal(out, oracle.topk(host(st.scores), cl, wl.topk, wl.offset))
