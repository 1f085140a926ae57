"""GPU parity of idx_publish_score, the decode step that publishes its
completed group's key and scores the cache including that key.  The
published row must equal the oracle's publish bit for bit, the scores of
positions [0, compress_lens) must equal the oracle's score of the updated
cache bit for bit (exact dots, the same fixed-order head sum), positions
past compress_lens stay unwritten, and the score histogram must count
exactly the scored positions.  Cases cover the single launch (new key at
T - 1: one extra workgroup per sequence), the two-launch form (new key
elsewhere, start_pos 0, Din past 2048), rows whose compress_lens stops
before the new key, a lone key (T = 1), 32 and 64 heads, and Din values
that take the 16-byte and the element loads.  The FP8 form
(idx_publish_score_fp8) equals its two calls bit for bit, and its published
row is the oracle's FP8 row of the oracle's key."""
import numpy as np
import pytest

import oracle
from sparse_attention_top_fp4_amd.inputs import YARN, normal_bf16, small_case

from gpu_util import bits, dev, host, say, sync, torch

pytestmark = pytest.mark.gpu

EPS = 1e-6
RATIO = 4
SENTINEL = np.float32(-12345.0)


@pytest.fixture(scope="module")
def idx():
    import sparse_attention_top_fp4_amd as m
    m.load_library()
    return m


def _counted_hist(scores_rows, counted):
    out = np.zeros((scores_rows.shape[0], 2048), np.int64)
    for r in range(scores_rows.shape[0]):
        v = scores_rows[r][counted[r]].astype(np.float32)
        v = np.where(v == 0.0, np.float32(0.0), v)
        u = v.view(np.uint32)
        key = np.where(u & 0x80000000, ~u, u | 0x80000000).astype(np.uint32)
        out[r] = np.bincount(key >> 21, minlength=2048)
    return out


CASES = [
    # (seed, B, H, T, tcap, Din, row, cl) -- row: the published cache row
    # (start_pos = ratio * row + ratio - 1, or 0 for "prefill-form" row 0);
    # cl None: every row scores [0, T)
    (91, 3, 64, 5000, 5000, 512, 4999, None),          # one launch, several chunks
    (92, 2, 32, 777, 800, 512, 776, None),             # ragged width, 32 heads, spare rows
    (93, 4, 64, 1, 1, 512, 0, None),                   # the new key alone
    (94, 3, 64, 3000, 3000, 512, 2999, [3000, 2999, 1500]),  # rows that stop before it
    (95, 2, 64, 70000, 70000, 512, 69999, None),       # long rows, many chunks
    (96, 2, 64, 2100, 2100, 203, 2099, None),          # element loads of wk
    (97, 2, 32, 1030, 1030, 2048, 1029, None),         # largest latent of the one launch
    (98, 2, 64, 1030, 1030, 2560, 1029, None),         # two launches: latent past 2048
    (99, 3, 64, 4000, 4096, 512, 3995, None),          # two launches: key not at T - 1
    (100, 2, 64, 1, 8, 512, "prefill-form", None),     # two launches: start_pos 0
]


@pytest.mark.parametrize("case", CASES)
def test_publish_score_matches_oracle(idx, case):
    t = torch()
    seed, B, H, T, tcap, din, row, cl = case
    say("publish+score", case)
    rng = np.random.default_rng(seed)
    c = small_case(seed, B, 1, H, T, tcap=tcap)
    start_pos = 0 if row == "prefill-form" else RATIO * row + RATIO - 1
    if cl is not None:
        c["cl"] = np.array(cl, np.int32)
    latent = normal_bf16(rng, (B, 1, din))
    wk = normal_bf16(rng, (128, din), std=0.02)
    gamma = (1.0 + 0.1 * rng.standard_normal(128)).astype(np.float32)
    P = max(start_pos + 1, 8)
    cs = oracle.yarn_cos_sin(P, 64, YARN["theta"], YARN["factor"], YARN["orig_len"],
                             YARN["beta_fast"], YARN["beta_slow"])
    kc0, _ = oracle.fp4_quant_rows(c["k"])
    kc_ref = kc0.copy()
    oracle.publish(latent, wk, gamma, cs, start_pos, RATIO, EPS, kc_ref)
    ref, _ = oracle.score(c["q"], c["w"], kc_ref, B, 1, H, T, c["cl"])

    kc = dev(kc0)
    sc = t.full((B, T + 3), float(SENTINEL), dtype=t.float32, device="cuda")
    hist = t.full((B, 2048), 5, dtype=t.int32, device="cuda")
    idx.idx_clear_key_hist(hist)
    idx.idx_publish_score(dev(latent), dev(wk), dev(gamma), dev(cs), start_pos, RATIO, EPS,
                          dev(c["q"]), dev(c["w"]), kc, T, dev(c["cl"]), sc, key_hist=hist)
    sync()
    assert np.array_equal(host(kc), kc_ref)
    got = host(sc)
    tt = np.arange(T)[None, :]
    live = tt < np.minimum(c["cl"], T)[:, None]
    assert np.array_equal(bits(got[:, :T][live]), bits(ref[live]))
    assert np.all(bits(got[:, :T][~live]) == bits(SENTINEL))
    assert np.all(bits(got[:, T:]) == bits(SENTINEL))
    assert np.array_equal(host(hist).astype(np.int64), _counted_hist(ref, live))


def test_publish_score_equals_two_calls(idx):
    """The single launch and idx_publish_keys followed by idx_score leave the
    same cache, scores and histogram, on a decode batch at the long-decode
    shape's per-row width with 64 heads."""
    t = torch()
    B, H, T = 4, 64, 16384
    say("publish+score vs two calls", B, H, T)
    rng = np.random.default_rng(120)
    c = small_case(120, B, 1, H, T)
    start_pos = RATIO * (T - 1) + RATIO - 1
    latent = dev(normal_bf16(rng, (B, 1, 512)))
    wk = dev(normal_bf16(rng, (128, 512), std=0.02))
    gamma = dev(np.ones(128, np.float32))
    cs = dev(oracle.yarn_cos_sin(start_pos + 1, 64, YARN["theta"], YARN["factor"],
                                 YARN["orig_len"], YARN["beta_fast"], YARN["beta_slow"]))
    kc0, _ = oracle.fp4_quant_rows(c["k"])
    q, w, cl = dev(c["q"]), dev(c["w"]), dev(c["cl"])
    outs = []
    for fused in (True, False):
        kc = dev(kc0)
        sc = t.full((B, T), float(SENTINEL), dtype=t.float32, device="cuda")
        hist = t.zeros((B, 2048), dtype=t.int32, device="cuda")
        if fused:
            idx.idx_publish_score(latent, wk, gamma, cs, start_pos, RATIO, EPS, q, w, kc, T, cl,
                                  sc, key_hist=hist)
        else:
            idx.idx_publish_keys(latent, wk, gamma, cs, start_pos, RATIO, EPS, kc)
            idx.idx_score(q, w, kc, B, 1, T, cl, sc, key_hist=hist)
        sync()
        outs.append((host(kc), bits(host(sc)), host(hist)))
    for a, b in zip(*outs):
        assert np.array_equal(a, b)


FP8_CASES = [
    # (seed, B, H, T, tcap, Din, row, cl), as CASES
    (131, 3, 64, 5000, 5000, 512, 4999, None),          # one launch, several chunks
    (132, 2, 32, 777, 800, 512, 776, None),             # 32 heads, spare rows
    (133, 2, 64, 1, 1, 512, 0, None),                   # the new key alone
    (134, 3, 64, 3000, 3000, 512, 2999, [3000, 2999, 1500]),  # rows that stop before it
    (135, 2, 64, 2100, 2100, 203, 2099, None),          # element loads of wk
    (136, 3, 64, 4000, 4096, 512, 3995, None),          # two launches: key not at T - 1
]


@pytest.mark.parametrize("case", FP8_CASES, ids=[str(c[0]) for c in FP8_CASES])
def test_publish_score_fp8_equals_two_calls(idx, case):
    """idx_publish_score_fp8 against idx_publish_keys_fp8 then idx_score_fp8:
    the same FP8 cache, scores and histogram bit for bit; the published row
    is the oracle's FP8 quantisation of the oracle's published key."""
    t = torch()
    seed, B, H, T, tcap, din, row, cl = case
    say("publish+score fp8", case)
    rng = np.random.default_rng(seed)
    c = small_case(seed, B, 1, H, T, tcap=tcap)
    if cl is not None:
        c["cl"] = np.array(cl, np.int32)
    start_pos = RATIO * row + RATIO - 1
    latent = normal_bf16(rng, (B, 1, din))
    wk = normal_bf16(rng, (128, din), std=0.02)
    gamma = (1.0 + 0.1 * rng.standard_normal(128)).astype(np.float32)
    cs = oracle.yarn_cos_sin(start_pos + 1, 64, YARN["theta"], YARN["factor"], YARN["orig_len"],
                             YARN["beta_fast"], YARN["beta_slow"])
    pre = oracle.publish(latent, wk, gamma, cs, start_pos, RATIO, EPS,
                         np.zeros((B, tcap, 68), np.uint8))
    want_row, _ = oracle.fp8_quant_rows(pre[:, 0])
    kc0, _ = oracle.fp8_quant_rows(c["k"])
    args = [dev(latent), dev(wk), dev(gamma), dev(cs)]
    q, w, cld = dev(c["q"]), dev(c["w"]), dev(c["cl"])
    outs = []
    for fused in (True, False):
        kc = dev(kc0)
        sc = t.full((B, T + 3), float(SENTINEL), dtype=t.float32, device="cuda")
        hist = t.zeros((B, 2048), dtype=t.int32, device="cuda")
        if fused:
            idx.idx_publish_score_fp8(*args, start_pos, RATIO, EPS, q, w, kc, T, cld, sc,
                                      key_hist=hist)
        else:
            idx.idx_publish_keys_fp8(*args, start_pos, RATIO, EPS, kc)
            idx.idx_score_fp8(q, w, kc, B, 1, T, cld, sc, key_hist=hist)
        sync()
        outs.append((host(kc), bits(host(sc)), host(hist)))
    for a, b in zip(*outs):
        assert np.array_equal(a, b)
    kc_got = outs[0][0]
    assert np.array_equal(kc_got[:, row], want_row)
    rest = np.ones(tcap, bool)
    rest[row] = False
    assert np.array_equal(kc_got[:, rest], kc0[:, rest])  # no other row written
    live = np.arange(T)[None, :] < np.minimum(c["cl"], T)[:, None]
    assert np.all(outs[0][1][:, :T][~live] == bits(SENTINEL))
    assert np.all(outs[0][1][:, T:] == bits(SENTINEL))
    assert outs[0][2].sum() == live.sum()


PAGE = 64
PAGE_STRIDE = PAGE * 68 + 128  # padded pages


def _paginate(kc_dev, seed, drop_last=()):
    """Scatter a contiguous device cache [B, T, 68] into a page pool with a
    padded stride, pages out of order and spare pages: (pages, block_table).
    Sequences in drop_last get an id past the pool for their last page."""
    t = torch()
    B, T, _ = kc_dev.shape
    npg = (T + PAGE - 1) // PAGE
    rng = np.random.default_rng(seed)
    n_pages = B * npg + 3
    perm = rng.permutation(n_pages)
    pages = t.zeros((n_pages, PAGE_STRIDE), dtype=t.uint8, device="cuda")
    bt = np.zeros((B, npg), np.int32)
    k = 0
    for b in range(B):
        for j in range(npg):
            p = int(perm[k])
            k += 1
            rows = kc_dev[b, j * PAGE:(j + 1) * PAGE].reshape(-1)
            pages[p, :rows.numel()] = rows
            bt[b, j] = p
        if b in drop_last:
            bt[b, npg - 1] = n_pages + 9
    return pages, dev(bt)


PAGED_CASES = [
    # (seed, B, H, T, Din, row, drop_last) -- row: the published cache row
    (131, 3, 64, 5000, 512, 4999, ()),        # one launch
    (132, 2, 32, 777, 203, 776, ()),          # ragged width, 32 heads, element loads
    (133, 4, 64, 16384, 512, 16383, (1,)),    # the new row's page missing in one sequence
    (134, 2, 64, 3000, 512, 2990, ()),        # two launches: key not at T - 1
]


@pytest.mark.parametrize("case", PAGED_CASES, ids=[str(c[0]) for c in PAGED_CASES])
def test_publish_score_paged_equals_contiguous_and_two_calls(idx, case):
    """idx_publish_score_paged leaves every page row, score and histogram
    count as idx_publish_keys_paged followed by idx_score_paged, and (with
    every page present) as the contiguous idx_publish_score and the
    oracle."""
    t = torch()
    seed, B, H, T, din, row, drop = case
    say("paged publish+score", case)
    rng = np.random.default_rng(seed)
    tcap = max(T, row + 1)
    c = small_case(seed, B, 1, H, T, tcap=tcap)
    start_pos = RATIO * row + RATIO - 1
    latent = dev(normal_bf16(rng, (B, 1, din)))
    wk = dev(normal_bf16(rng, (128, din), std=0.02))
    gamma = dev((1.0 + 0.1 * rng.standard_normal(128)).astype(np.float32))
    cs = dev(oracle.yarn_cos_sin(start_pos + 1, 64, YARN["theta"], YARN["factor"],
                                 YARN["orig_len"], YARN["beta_fast"], YARN["beta_slow"]))
    kc0, _ = oracle.fp4_quant_rows(c["k"])
    q, w, cl = dev(c["q"]), dev(c["w"]), dev(c["cl"])
    outs = []
    for fused in (True, False):
        pages, bt = _paginate(dev(kc0), seed, drop)
        sc = t.full((B, T), float(SENTINEL), dtype=t.float32, device="cuda")
        hist = t.zeros((B, 2048), dtype=t.int32, device="cuda")
        if fused:
            idx.idx_publish_score_paged(latent, wk, gamma, cs, start_pos, RATIO, EPS, q, w, pages,
                                        bt, T, cl, sc, key_hist=hist)
        else:
            idx.idx_publish_keys_paged(latent, wk, gamma, cs, start_pos, RATIO, EPS, pages, bt,
                                       tcap)
            idx.idx_score_paged(q, w, pages, bt, B, 1, T, cl, sc, key_hist=hist)
        sync()
        outs.append((host(pages), bits(host(sc)), host(hist)))
    for a, b in zip(*outs):
        assert np.array_equal(a, b)
    if not drop:
        kc = dev(kc0)
        sc = t.full((B, T), float(SENTINEL), dtype=t.float32, device="cuda")
        hist = t.zeros((B, 2048), dtype=t.int32, device="cuda")
        idx.idx_publish_score(latent, wk, gamma, cs, start_pos, RATIO, EPS, q, w, kc, T, cl, sc,
                              key_hist=hist)
        sync()
        assert np.array_equal(outs[0][1], bits(host(sc)))
        assert np.array_equal(outs[0][2], host(hist))
