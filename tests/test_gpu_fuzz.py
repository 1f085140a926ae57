"""Seeded fuzz of the score and top-k entry points against the oracle:
random shapes (32 or 64 heads, ragged T, padded strides), compress_lens
anywhere in [-2, T + 3] (the kernels clamp it to [0, T]), index_topk below
and above T, offsets of both signs.  Every case runs each path a caller can
take to the indices:
  idx_score (+ histogram) -> idx_topk, idx_topk without the histogram,
  idx_score_topk with and without scores, idx_score_topk_q4 on the
  quantiser's rows;
scores bit-identical below compress_lens, indices bit-exact."""
import numpy as np
import pytest

import oracle
from sparse_attention_top_fp4_amd.inputs import small_case

from gpu_util import bits, dev, fp4_cache, host, say, sync, torch

pytestmark = pytest.mark.gpu

N_CASES = 24


@pytest.fixture(scope="module")
def idx():
    import sparse_attention_top_fp4_amd as m
    m.load_library()
    return m


def _draw(i):
    rng = np.random.default_rng(5000 + i)
    H = int(rng.choice([32, 64]))
    B = int(rng.integers(1, 4))
    S = int(rng.integers(1, 7))
    T = int(rng.integers(1, 2600)) if i % 6 else int(rng.integers(1, 70))
    tcap = T + int(rng.integers(0, 40))
    c = small_case(6000 + i, B, S, H, T, start_pos=0 if S > 1 else None, tcap=tcap)
    R = B * S
    cl = rng.integers(-2, T + 4, size=R).astype(np.int32)
    cl[0] = T
    if R > 1:
        cl[1] = 0
    if i % 4 == 0:  # a causal pattern instead
        cl = c["cl"].copy()
    c["cl"] = cl
    k = int(rng.integers(1, T + 50))
    offset = int(rng.integers(-1000, 1000))
    pad = int(rng.integers(0, 9))
    return c, B, S, H, T, k, offset, pad


@pytest.mark.parametrize("i", range(N_CASES))
def test_fuzz_score_and_topk(idx, i):
    t = torch()
    c, B, S, H, T, k, offset, pad = _draw(i)
    R = B * S
    say("fuzz", i, dict(B=B, S=S, H=H, T=T, k=k, offset=offset, pad=pad))
    kc_ref, _ = oracle.fp4_quant_rows(c["k"])
    ref, inexact = oracle.score(c["q"], c["w"], kc_ref, B, S, H, T, c["cl"])
    assert inexact == 0
    ref_idx = oracle.topk(ref, c["cl"], k, offset)
    kout = min(k, T)
    lim = np.clip(c["cl"], 0, T)

    kc = fp4_cache(c["k"])
    q, w, cl = dev(c["q"]), dev(c["w"]), dev(c["cl"])
    ld = T + pad
    sc = t.full((R, ld), float("nan"), dtype=t.float32, device="cuda")
    hist = t.empty((R, 2048), dtype=t.int32, device="cuda")
    idx.idx_clear_key_hist(hist)
    idx.idx_score(q, w, kc, B, S, T, cl, sc, key_hist=hist)
    out_h = t.full((R, kout + 2), -7, dtype=t.int32, device="cuda")
    idx.idx_topk(sc, T, cl, k, offset, out_h, key_hist=hist)
    out_p = t.full((R, kout + 2), -7, dtype=t.int32, device="cuda")
    idx.idx_topk(sc, T, cl, k, offset, out_p)
    out_f = t.full((R, kout + 2), -7, dtype=t.int32, device="cuda")
    idx.idx_score_topk(q, w, kc, B, S, T, cl, k, offset, out_f)
    sc_f = t.full((R, ld), float("nan"), dtype=t.float32, device="cuda")
    out_fs = t.full((R, kout + 2), -7, dtype=t.int32, device="cuda")
    idx.idx_score_topk(q, w, kc, B, S, T, cl, k, offset, out_fs, scores=sc_f)
    rows = t.empty((R, H, 68), dtype=t.uint8, device="cuda")
    idx.idx_fp4_quant(q, rows)
    out_q4 = t.full((R, kout + 2), -7, dtype=t.int32, device="cuda")
    idx.idx_score_topk_q4(rows, w, kc, B, S, T, cl, k, offset, out_q4)
    sync()

    g, gf = host(sc), host(sc_f)
    for r in range(R):
        n = int(lim[r])
        assert np.array_equal(bits(g[r, :n]), bits(ref[r, :n])), ("idx_score", r)
        assert np.array_equal(bits(gf[r, :n]), bits(ref[r, :n])), ("idx_score_topk", r)
    assert np.all(np.isnan(g[:, T:])) and np.all(np.isnan(gf[:, T:]))
    assert not host(hist).any()  # consumed and reset by idx_topk
    for name, o in (("topk+hist", out_h), ("topk", out_p), ("fused", out_f),
                    ("fused+scores", out_fs), ("fused q4", out_q4)):
        got = host(o)
        assert np.array_equal(got[:, :kout], ref_idx), name
        assert np.all(got[:, kout:] == -7), name
