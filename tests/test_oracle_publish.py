"""Pins of the oracle's key publish and RoPE table.

Publish definition: "DeepSeek V4.1" page, class Indexer, forward (k =
k_norm(wk(latent)), RoPE on the last rope_head_dim dims at the group's
position, fp4 round trip, write into k_cache at start_pos // ratio).  RoPE
table: "Module compress" page, yarn_freqs_cis (YaRN; its constants are not
printed, so their values are a reading; the table's construction is pinned by
the correction-dimension equation, a hand-worked band and hand-worked ramp
values).
"""
import math

import numpy as np

import oracle
from sparse_attention_top_fp4_amd.inputs import YARN, bf16_to_f32, normal_bf16


def _inputs(seed, B=3, G=1, din=512):
    rng = np.random.default_rng(seed)
    latent = normal_bf16(rng, (B, G, din))
    wk = normal_bf16(rng, (128, din), std=0.02)
    gamma = np.ones(128, np.float32)
    return latent, wk, gamma


def _ref64(latent, wk, gamma, cs_row, eps, rd=64):
    """float64 restatement without intermediate rounding."""
    y = bf16_to_f32(wk).astype(np.float64) @ bf16_to_f32(latent).astype(np.float64)
    z = y / np.sqrt(np.mean(y * y) + eps) * gamma.astype(np.float64)
    base = 128 - rd
    x = z[base:].reshape(-1, 2)
    c, s = cs_row[:, 0].astype(np.float64), cs_row[:, 1].astype(np.float64)
    rot = (x[:, 0] + 1j * x[:, 1]) * (c + 1j * s)  # textbook complex rotation
    z = z.copy()
    z[base::2] = rot.real
    z[base + 1::2] = rot.imag
    return z


def test_yarn_factor_one_is_plain_rope():
    P, rd, theta = 4000, 64, 10000.0
    t = oracle.yarn_cos_sin(P, rd, theta, 1.0, 0, 32.0, 1.0)
    i = np.arange(rd // 2)
    ang = np.arange(P)[:, None] * theta ** (-(2.0 * i) / rd)[None, :]
    assert np.allclose(t[..., 0], np.cos(ang), atol=1e-6, rtol=0)
    assert np.allclose(t[..., 1], np.sin(ang), atol=1e-6, rtol=0)
    assert np.all(t[0, :, 0] == 1.0) and np.all(t[0, :, 1] == 0.0)


def test_yarn_correction_dim_meets_its_definition():
    """The correction dimension d(beta) is where a pair turns beta times over
    the original context: orig_len * theta^(-2d/rd) / (2 pi) == beta."""
    for beta in (YARN["beta_fast"], YARN["beta_slow"], 4.0, 0.5):
        for rd, theta, orig in ((64, YARN["theta"], YARN["orig_len"]), (128, 50000.0, 4096)):
            d = oracle.yarn_correction_dim(beta, rd, theta, orig)
            turns = orig * theta ** (-2.0 * d / rd) / (2.0 * math.pi)
            assert abs(turns / beta - 1.0) < 1e-12


def test_yarn_band_hand_worked():
    """Band of the chosen constants (theta 1e4, rd 64, original length 65536,
    beta 32 / 1), worked by hand:
      d(32) = 32 * ln(65536 / (64 pi)) / ln(1e4) = 32 * 5.78673 / 9.21034 = 20.105
      d(1)  = 32 * ln(65536 / (2 pi))  / ln(1e4) = 32 * 9.25250 / 9.21034 = 32.146
    so lo = floor(20.105) = 20 and hi = ceil(32.146) = 33, inside [0, rd - 1]
    (a clamp at rd/2 - 1 would have cut hi to 31)."""
    assert oracle.yarn_correction_range(64, YARN["theta"], YARN["orig_len"], YARN["beta_fast"],
                                        YARN["beta_slow"]) == (20, 33)
    # clamps: a short original length puts d(beta_fast) below 0, a long one
    # puts d(beta_slow) beyond rd - 1
    assert oracle.yarn_correction_range(64, 1e4, 100, 32.0, 1.0)[0] == 0
    assert oracle.yarn_correction_range(16, 1e4, 10 ** 9, 32.0, 1.0)[1] == 15


def test_yarn_ramp_hand_worked():
    """Frequency of pair i over its plain value, for the band [20, 33] and
    factor 16: 1 for i <= 20; 1 - (15/16)(i - 20)/13 inside (i = 26: 118/208,
    i = 31: 43/208).  Read back from the table's angle at position 1."""
    rd = 64
    t = oracle.yarn_cos_sin(2, rd, YARN["theta"], YARN["factor"], YARN["orig_len"],
                            YARN["beta_fast"], YARN["beta_slow"])
    f = np.arctan2(t[1, :, 1].astype(np.float64), t[1, :, 0].astype(np.float64))
    plain = YARN["theta"] ** (-(2.0 * np.arange(rd // 2)) / rd)
    r = f / plain
    assert np.all(np.abs(r[:21] - 1.0) < 1e-6)
    assert abs(r[26] - 118.0 / 208.0) < 1e-6
    assert abs(r[31] - 43.0 / 208.0) < 1e-5
    assert np.all(np.diff(r) <= 1e-6)
    f64 = oracle.yarn_frequencies(rd, YARN["theta"], YARN["factor"], YARN["orig_len"],
                                  YARN["beta_fast"], YARN["beta_slow"])
    assert f64[20] == plain[20] and abs(f64[26] / plain[26] - 118.0 / 208.0) < 1e-15


def test_prequant_key_matches_float64_within_bf16_rounding():
    latent, wk, gamma = _inputs(1)
    P = 4096
    cs = oracle.yarn_cos_sin(P, 64, YARN["theta"], YARN["factor"], YARN["orig_len"],
                             YARN["beta_fast"], YARN["beta_slow"])
    start_pos, ratio = 4 * 700 - 1, 4
    kc = np.zeros((3, 800, 68), np.uint8)
    pre = oracle.publish(latent, wk, gamma, cs, start_pos, ratio, 1e-6, kc)
    pos = start_pos + 1 - ratio
    for b in range(3):
        ref = _ref64(latent[b, 0], wk, gamma, cs[pos], 1e-6)
        got = bf16_to_f32(pre[b, 0]).astype(np.float64)
        pair = np.repeat(np.sqrt(ref[0::2] ** 2 + ref[1::2] ** 2), 2)
        assert np.all(np.abs(got - ref) <= 2.0 ** -6 * pair + 1e-6)
        assert abs(np.mean(ref * ref) - 1.0) < 1e-3  # RMSNorm with gamma = 1
    # only row start_pos // ratio of each sequence was written, with the
    # oracle's own quantisation of the pre-quantisation key
    written = np.flatnonzero(kc.reshape(3 * 800, 68).any(axis=1))
    assert list(written) == [b * 800 + 699 for b in range(3)]
    rows, _ = oracle.fp4_quant_rows(pre[:, 0])
    assert np.array_equal(kc[:, 699], rows)


def test_rope_identity_at_position_zero_and_norm_preservation():
    latent, wk, gamma = _inputs(2, B=2, G=3)
    P = 64
    cs = oracle.yarn_cos_sin(P, 64, YARN["theta"], YARN["factor"], YARN["orig_len"],
                             YARN["beta_fast"], YARN["beta_slow"])
    ident = np.zeros_like(cs)
    ident[..., 0] = 1.0
    kc = np.zeros((2, 16, 68), np.uint8)
    pre = oracle.publish(latent, wk, gamma, cs, 0, 4, 1e-6, kc)  # prefill: group g at pos 4g
    kc2 = np.zeros_like(kc)
    pre_id = oracle.publish(latent, wk, gamma, ident, 0, 4, 1e-6, kc2)
    assert np.array_equal(pre[:, 0], pre_id[:, 0])  # position 0 rotates by nothing
    assert not np.array_equal(pre[:, 1], pre_id[:, 1])
    a = bf16_to_f32(pre[:, 1:, 64:]).astype(np.float64).reshape(-1, 2)
    b = bf16_to_f32(pre_id[:, 1:, 64:]).astype(np.float64).reshape(-1, 2)
    na, nb = np.hypot(a[:, 0], a[:, 1]), np.hypot(b[:, 0], b[:, 1])
    assert np.all(np.abs(na - nb) <= 2.0 ** -7 * nb + 1e-6)
    assert np.array_equal(pre[:, :, :64], pre_id[:, :, :64])  # the non-RoPE part is untouched
    written = np.flatnonzero(kc.reshape(-1, 68).any(axis=1))
    assert list(written) == [0, 1, 2, 16, 17, 18]
