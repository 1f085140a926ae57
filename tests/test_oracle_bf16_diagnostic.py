"""Diagnostic (reported, not gating): how far the fp32 score contract's
selections are from the page's own bf16 tensor pipeline ("DeepSeek V4.1"
page, class Indexer, forward: einsum, relu_, times weights, sum over heads
as bf16 tensors; "Module compress" page, precision: the scores are bf16
tensors).  The bf16 scores tie often, so the two top-k sets differ at the
threshold; the overlap is printed for the tiny decode workload and sampled
rows of the batched decode at 128K, and must stay high.

Pins of the literal pipeline itself: the fp4 row decoding equals the
quantiser's round trip, and one head with unit weight gives bf16(relu(dot))."""
import numpy as np

import oracle
from sparse_attention_top_fp4_amd.inputs import bf16_bits, generate, normal_bf16, workload


def test_row_decoding_equals_round_trip():
    rng = np.random.default_rng(2)
    x = normal_bf16(rng, (50, 128))
    rows, rt = oracle.fp4_quant_rows(x)
    dec = oracle._dequant_rows(rows)
    assert np.array_equal(bf16_bits(dec), rt)


def test_single_head_is_bf16_relu_dot():
    rng = np.random.default_rng(4)
    q = normal_bf16(rng, (1, 1, 128))
    k = normal_bf16(rng, (1, 64, 128))
    kc, _ = oracle.fp4_quant_rows(k)
    d, _ = oracle.head_dots(q, kc, 1, 1, 1, 64)
    w = bf16_bits(np.ones((1, 1), np.float32))
    s = oracle.score_bf16_literal(q, w, kc, 1, 1, 64, np.array([64], np.int32))
    assert np.array_equal(s[0], oracle._bf16_round(np.maximum(oracle._bf16_round(d[0, 0]), 0)))


def _overlap(cid, rows):
    wl = workload(cid)
    inp = generate(wl, rows=set(rows // wl.S))
    kc, _ = oracle.fp4_quant_rows(inp["k"])
    sel = rows
    q, w, cl = inp["q"][sel], inp["w"][sel], inp["cl"][sel]
    s32, _ = oracle.score(q, w, kc, len(sel), 1, wl.H, wl.T, cl)
    s16 = oracle.score_bf16_literal(q, w, kc, 1, wl.H, wl.T, cl)
    ties = float(np.mean([1 - len(np.unique(r[np.isfinite(r)])) / np.isfinite(r).sum()
                          for r in s16]))
    return oracle.topk_overlap(s32, s16, cl, wl.topk), ties


def test_bf16_pipeline_overlap_tiny_decode():
    ov, ties = _overlap(0, np.array([0]))
    print(f"[bf16 diagnostic] tiny_decode: top-256 overlap {ov:.4f}, bf16 tie share {ties:.3f}")
    assert ov >= 0.9


def test_bf16_pipeline_overlap_batched_decode_sample():
    ov, ties = _overlap(1, np.array([0, 1]))
    print(f"[bf16 diagnostic] batched_decode_128k rows 0-1: top-2048 overlap {ov:.4f}, "
          f"bf16 tie share {ties:.3f}")
    assert ov >= 0.9
