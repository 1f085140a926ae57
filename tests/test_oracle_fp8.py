"""Pins of the oracle's FP8 indexer cache (no GPU).

Row format: [VLLM] "attention.py" patch, _indexer_k_cache_head_dim (128 fp8
bytes and one fp32 scale per 128 values, 132 bytes) and
DeepseekV4Indexer.__init__ (quant_block_size 128, scale_fmt "ue8m0").  Read
here as OCP e4m3 codes with a power-of-two scale 2^e, e the smallest integer
with 448 * 2^e >= amax (amax at least 448 * 2^-126), values rounded to the
nearest e4m3 point of x / 2^e with ties to the even code.

- the e4m3 values the oracle produces equal the format's definition, for
  every one of the 127 finite non-negative codes (and their negatives);
- the scale exponent over every finite bf16 amax, against exact rationals;
- the hand-worked tie table tests/golden/e4m3_rne_ties.txt;
- the nearest-point property over every finite bf16 input at scale 2^0;
- the per-head dot equals the float64 product of the dequantised rows,
  rounded once to fp32;
- the score on fp4 round trips with equal block scales (exactly
  representable in e4m3) equals the fp4 score bit for bit.
"""
import os
from fractions import Fraction

import numpy as np

import oracle
from sparse_attention_top_fp4_amd.inputs import bf16_bits, bf16_to_f32, head_weights, normal_bf16

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "e4m3_rne_ties.txt")


def e4m3_def(c):
    """OCP e4m3 value of code c (0..255, c & 0x7f != 0x7f)."""
    s, E, m = c >> 7, (c >> 3) & 15, c & 7
    v = m * 2.0 ** -9 if E == 0 else (8 + m) * 2.0 ** (E - 10)
    return -v if s else v


FINITE_POS = [c for c in range(127)]  # 0x7f is NaN


def _blocks(values, first=448.0):
    """Rows of 128 bf16 values: `first`, then values (zero padded)."""
    vals = np.asarray(values, np.float32)
    n = -(-len(vals) // 127)
    x = np.zeros((n, 128), np.float32)
    x[:, 0] = first
    flat = x[:, 1:].reshape(-1)
    flat[:len(vals)] = vals
    x[:, 1:] = flat.reshape(n, 127)
    return bf16_bits(x)


def test_code_values_match_the_format():
    vals = [e4m3_def(c) for c in FINITE_POS]
    assert max(vals) == 448.0 and vals == sorted(vals)
    x = _blocks(vals + [-v for v in vals])
    rows, rt = oracle.fp8_quant_rows(x)
    assert np.all(rows[:, 128:].view(np.float32) == 1.0)  # scale 2^0
    got_codes = rows[:, 1:128].reshape(-1)[:2 * len(vals)]
    want = np.array(FINITE_POS + [c | 0x80 for c in FINITE_POS], np.uint8)
    # -0 keeps its sign: code 0x80
    assert np.array_equal(got_codes, want)
    assert np.array_equal(bf16_to_f32(rt[:, 1:128].reshape(-1)[:2 * len(vals)]),
                          np.array(vals + [-v for v in vals], np.float32))


def test_scale_exponent_exhaustive_over_bf16():
    pats = np.arange(0x0001, 0x7F80, dtype=np.uint32).astype(np.uint16)  # positive finite
    x = np.zeros((len(pats), 128), np.uint16)
    x[:, 0] = pats
    rows, _ = oracle.fp8_quant_rows(x)
    scale = rows[:, 128:].copy().view(np.float32)[:, 0]
    amax = bf16_to_f32(pats).astype(np.float64)
    floor_ = Fraction(448) * Fraction(2) ** -126
    for i in range(0, len(pats), 97):  # exact rationals on a spread of amax values
        a = max(Fraction(float(amax[i])), floor_)
        s = Fraction(float(scale[i]))
        assert 448 * s >= a and 448 * s / 2 < a, (hex(pats[i]), float(scale[i]))
    # and the power-of-two ceiling in closed form on every one of them
    a = np.maximum(amax, 448.0 * 2.0 ** -126)
    e = np.ceil(np.log2(a / 448.0))
    assert np.array_equal(scale.astype(np.float64), 2.0 ** e)


def test_tie_table_golden():
    rows = []
    for line in open(GOLDEN):
        line = line.split("#")[0].strip()
        if line:
            x, v, c = line.split()[:3]
            rows.append((float(x), float(v), int(c, 16)))
    x = np.zeros((1, 128), np.float32)
    for i, (xi, _, _) in enumerate(rows):
        x[0, i] = xi
    q, rt = oracle.fp8_quant_rows(bf16_bits(x))
    for i, (xi, v, c) in enumerate(rows):
        assert q[0, i] == c, (xi, hex(q[0, i]), hex(c))
        got = bf16_to_f32(rt[0, i:i + 1])[0]
        assert got == v and np.signbit(got) == np.signbit(v), (xi, got, v)


def test_nearest_point_over_every_bf16():
    pats = np.arange(0x10000, dtype=np.uint32).astype(np.uint16)
    xs = bf16_to_f32(pats)
    keep = np.isfinite(xs) & (np.abs(xs) <= 448.0)
    xs = xs[keep]
    rows, rt = oracle.fp8_quant_rows(_blocks(xs))
    got = bf16_to_f32(rt[:, 1:128].reshape(-1)[:len(xs)]).astype(np.float64)
    table = np.array(sorted({abs(e4m3_def(c)) for c in FINITE_POS}), np.float64)
    y = np.abs(xs.astype(np.float64))
    j = np.clip(np.searchsorted(table, y), 1, len(table) - 1)
    best = np.minimum(np.abs(y - table[j - 1]), np.abs(y - table[j]))
    assert np.all(np.abs(np.abs(got) - y) == best)
    assert np.all((got == 0) | (np.sign(got) == np.sign(xs)))


def test_head_dots_equal_float64_product():
    rng = np.random.default_rng(3)
    q = normal_bf16(rng, (2, 4, 128))
    k = normal_bf16(rng, (1, 37, 128))
    k[0, 5] = bf16_bits(np.float32(1e-3) * bf16_to_f32(k[0, 5]))  # a small row
    kc, krt = oracle.fp8_quant_rows(k)
    _, qrt = oracle.fp8_quant_rows(q)
    d, _ = oracle.head_dots_fp8(q, kc, 1, 2, 4, 37)
    ref = np.einsum("rhd,td->rht", bf16_to_f32(qrt).astype(np.float64),
                    bf16_to_f32(krt[0]).astype(np.float64))
    assert np.array_equal(d, ref.astype(np.float32))


def test_score_equals_fp4_score_on_shared_grid():
    """fp4 round trips whose four block scales are equal are exactly
    representable in e4m3 at one block-128 scale (the e2m1 grid times 2^e is
    {0, 32, ..., 384} times 2^(e-6)), so both scores use the same exact dots
    and the same head order."""
    rng = np.random.default_rng(11)
    B, S, H, T = 2, 3, 64, 40

    def equal_scale_rt(x):
        x = bf16_to_f32(x).copy()
        x[..., ::32] = 5.5  # every 32-block has the same amax, so the same scale
        _, rt = oracle.fp4_quant_rows(bf16_bits(x))
        return rt

    q = equal_scale_rt(normal_bf16(rng, (B * S, H, 128)))
    k = equal_scale_rt(normal_bf16(rng, (B, T, 128)))
    w = head_weights(rng, B * S, H)
    cl = np.array([40, 17, 0, 40, 39, 1], np.int32)
    kc4, _ = oracle.fp4_quant_rows(k)
    kc8, krt8 = oracle.fp8_quant_rows(k)
    assert np.array_equal(krt8, k)  # lossless in e4m3
    s4, n4 = oracle.score(q, w, kc4, B, S, H, T, cl)
    s8, _ = oracle.score_fp8(q, w, kc8, B, S, H, T, cl)
    assert n4 == 0
    assert np.array_equal(s4.view(np.uint32), s8.view(np.uint32))
    cand = np.array([[0, 3], [1, 2], [0, 0], [4, 4], [2, 3], [0, 1]], np.int32)
    s4c, _ = oracle.score(q, w, kc4, B, S, H, T, cl, cand=cand, cbs=8)
    s8c, _ = oracle.score_fp8(q, w, kc8, B, S, H, T, cl, cand=cand, cbs=8)
    assert np.array_equal(s4c.view(np.uint32), s8c.view(np.uint32))


def test_score_single_head_is_relu_dot():
    rng = np.random.default_rng(5)
    q = normal_bf16(rng, (1, 1, 128))
    k = normal_bf16(rng, (1, 50, 128))
    kc, _ = oracle.fp8_quant_rows(k)
    d, _ = oracle.head_dots_fp8(q, kc, 1, 1, 1, 50)
    w = bf16_bits(np.ones((1, 1), np.float32))
    s, _ = oracle.score_fp8(q, w, kc, 1, 1, 1, 50, np.array([50], np.int32))
    assert np.array_equal(s[0], np.maximum(d[0, 0], 0.0) + np.float32(0.0))
