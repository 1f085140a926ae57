"""Pins of the oracle's fp4 quantiser against what the pages fix.

The pages state the rule in words ("Module compress" page: fp4_quant_e8m0_inplace
and to_e2m1_rne; the 68-byte row of the vLLM attention.py page,
_indexer_k_cache_head_dim).  Each test checks the oracle against an
independent statement of that rule: exact rationals for the scale, a
hand-written tie table, and properties (nearest point, idempotence, range).
"""
import os
from fractions import Fraction

import numpy as np

import oracle
from sparse_attention_top_fp4_amd.inputs import bf16_bits, bf16_to_f32

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def _finite_positive_bf16():
    b = np.arange(1, 0x7F80, dtype=np.uint16)  # +subnormals .. max finite
    return b


def _rows_with_block0(vals_bits, fill_bits=None):
    """One 128-wide row per value: block 0 = [v, fill...], other blocks 0."""
    n = len(vals_bits)
    x = np.zeros((n, 128), np.uint16)
    x[:, 0] = vals_bits
    if fill_bits is not None:
        x[:, 1] = fill_bits
    return x


def _exact_e(a: Fraction) -> int:
    """Smallest integer e with 6*2^e >= max(a, 6*2^-126), by exact rationals."""
    a = max(a, Fraction(6) * Fraction(1, 2 ** 126))
    e = int(np.floor(np.log2(float(a) / 6.0))) - 2
    while Fraction(6) * (Fraction(2) ** e) < a:
        e += 1
    return e


def test_e8m0_scale_exhaustive_over_bf16_amax():
    bits = _finite_positive_bf16()
    rows, _ = oracle.fp4_quant_rows(_rows_with_block0(bits))
    got = rows[:, 64].astype(int) - 127
    vals = bf16_to_f32(bits).astype(np.float64)
    exp = np.array([_exact_e(Fraction(float(v))) for v in vals])
    assert np.array_equal(got, exp)
    # sign of the maximum does not matter
    rows_neg, _ = oracle.fp4_quant_rows(_rows_with_block0(bits | np.uint16(0x8000)))
    assert np.array_equal(rows_neg[:, 64], rows[:, 64])
    # the all-zero blocks 1..3 take the floor: e = -126, byte 1
    assert np.all(rows[:, 65:68] == 1)


def test_e8m0_boundaries():
    # amax = 3*2^(k+1) = 6*2^k gives exactly e = k; the next bf16 up gives k+1
    for k in (-126, -100, -3, 0, 1, 7, 60, 124):
        a = np.float32(6.0 * 2.0 ** k)
        ab = bf16_bits(np.array([a]))
        up = ab + np.uint16(1)
        rows, _ = oracle.fp4_quant_rows(_rows_with_block0(np.concatenate([ab, up])))
        assert int(rows[0, 64]) - 127 == k
        assert int(rows[1, 64]) - 127 == k + 1


def test_e2m1_tie_table_golden():
    vals, codes = [], []
    for line in open(os.path.join(GOLDEN, "e2m1_rne_ties.txt")):
        line = line.split("#")[0].strip()
        if not line:
            continue
        v, c = line.split()
        vals.append(float(v))
        codes.append(int(c))
    vals = np.array(vals, np.float32)
    x = np.zeros((len(vals), 128), np.uint16)
    x[:, 0] = bf16_bits(vals)
    x[:, 1] = bf16_bits(np.array([6.0], np.float32))[0]  # fixes the scale at 2^0
    rows, rt = oracle.fp4_quant_rows(x)
    assert np.all(rows[:, 64] == 127)
    got = rows[:, 0] & 0xF
    assert list(got) == codes
    # the 68-byte layout: element 1 (value 6.0 -> code 7) is the high nibble of byte 0
    assert np.all(rows[:, 0] >> 4 == 7)


def test_e2m1_neighbours_of_midpoints_round_to_nearest():
    mids = [(0.25, 0, 1), (0.75, 1, 2), (1.25, 2, 3), (1.75, 3, 4), (2.5, 4, 5), (3.5, 5, 6),
            (5.0, 6, 7)]
    six = bf16_bits(np.array([6.0], np.float32))[0]
    for m, lo, hi in mids:
        mb = bf16_bits(np.array([m], np.float32))[0]
        x = np.zeros((2, 128), np.uint16)
        x[:, 1] = six
        x[0, 0] = mb - 1  # next bf16 below the midpoint
        x[1, 0] = mb + 1  # next bf16 above
        rows, _ = oracle.fp4_quant_rows(x)
        assert (rows[0, 0] & 0xF) == lo and (rows[1, 0] & 0xF) == hi, m


def _decode_codes(rows):
    lo = rows[..., :64] & 0xF
    hi = rows[..., :64] >> 4
    codes = np.empty(rows.shape[:-1] + (128,), np.uint8)
    codes[..., 0::2] = lo
    codes[..., 1::2] = hi
    return codes


def test_nearest_point_property_all_bf16():
    """Every finite bf16 value, quantised in blocks of scale 2^e for several
    e: the chosen grid point is at minimal distance, a tie takes the even
    code, the sign bit is the input's, and the round trip is code*2^e."""
    allb = np.arange(0, 0x10000, dtype=np.uint32).astype(np.uint16)
    finite = (allb & 0x7F80) != 0x7F80
    allb = allb[finite]
    for e in (-126, -20, 0, 9, 125):
        amax = np.float32(6.0 * 2.0 ** e)
        mag = np.abs(bf16_to_f32(allb).astype(np.float64))
        sel = allb[mag <= float(amax)]
        n = len(sel)
        pad = (-n) % 31
        sel = np.concatenate([sel, np.zeros(pad, np.uint16)])
        blocks = sel.reshape(-1, 31)
        amaxb = bf16_bits(np.array([amax]))[0]
        x = np.concatenate([blocks, np.full((blocks.shape[0], 1), amaxb, np.uint16)], axis=1)
        nrow = (x.shape[0] + 3) // 4
        xx = np.zeros((nrow * 4, 32), np.uint16)
        xx[: x.shape[0]] = x
        xx[x.shape[0]:, 31] = amaxb
        xx = xx.reshape(nrow, 128)
        rows, rt = oracle.fp4_quant_rows(xx)
        assert np.all(rows[:, 64:].astype(int) - 127 == e)
        codes = _decode_codes(rows).reshape(-1)
        v = bf16_to_f32(xx.reshape(-1)).astype(np.float64)
        y = np.abs(v) * 2.0 ** (-e)
        mag_code = codes & 7
        dist = np.abs(y[:, None] - GRID[None, :])
        chosen = dist[np.arange(len(y)), mag_code]
        best = dist.min(axis=1)
        assert np.all(chosen == best)
        n_best = (dist == best[:, None]).sum(axis=1)
        assert np.all((n_best == 1) | (mag_code % 2 == 0))
        assert np.array_equal((codes >> 3).astype(bool), np.signbit(v))
        back = np.where(codes >> 3, -1.0, 1.0) * GRID[mag_code] * 2.0 ** e
        assert np.array_equal(bf16_to_f32(rt.reshape(-1)).astype(np.float64), back)


def test_scaled_amax_in_range_and_idempotence():
    rng = np.random.default_rng(5)
    for std in (1e-30, 1e-3, 1.0, 1e3, 1e30):
        x = bf16_bits(rng.standard_normal((257, 128)).astype(np.float32) * np.float32(std))
        rows, rt = oracle.fp4_quant_rows(x)
        v = bf16_to_f32(x).astype(np.float64).reshape(-1, 4, 32)
        amax = np.abs(v).max(axis=2)
        e = rows[:, 64:].astype(int) - 127
        ratio = amax / 2.0 ** e
        ok = amax > 6.0 * 2.0 ** -126
        assert np.all((ratio[ok] > 3.0) & (ratio[ok] <= 6.0))
        # the round trip is idempotent in value (a block whose maximum rounded
        # down may re-encode with a halved scale and doubled codes)
        rows2, rt2 = oracle.fp4_quant_rows(rt)
        assert np.array_equal(rt2, rt)


def test_zero_blocks():
    x = np.zeros((2, 128), np.uint16)
    x[1, :] = 0x8000  # all -0
    rows, rt = oracle.fp4_quant_rows(x)
    assert np.all(rows[:, 64:] == 1)  # e = -126
    assert np.all(rows[0, :64] == 0)
    assert np.all(rows[1, :64] == 0x88)
    assert np.array_equal(rt, x)
