"""Pins of the oracle's query step: RoPE on the query heads, fp4 quantise,
weight scaling.

Definition: "DeepSeek V4.1" page, class Indexer, forward (q split into
index_n_heads heads, apply_rotary_emb on the last rope_head_dim dims at
positions start_pos..end_pos, fp4_act_quant, weights = weights_proj(x) *
softmax_scale * n_heads^-0.5); the vLLM attention.py page fuses the three as
fused_indexer_q_rope_quant.  The RoPE table is an input (its YaRN constants
are parity unpinned, as for the key publish).
"""
import numpy as np

import oracle
from sparse_attention_top_fp4_amd.inputs import YARN, bf16_bits, bf16_to_f32, normal_bf16


def _table(P):
    return oracle.yarn_cos_sin(P, 64, YARN["theta"], YARN["factor"], YARN["orig_len"],
                               YARN["beta_fast"], YARN["beta_slow"])


def _case(seed, B=2, S=5, H=8):
    rng = np.random.default_rng(seed)
    q = normal_bf16(rng, (B * S, H, 128))
    w = normal_bf16(rng, (B * S, H))
    return q, w


def test_position_zero_and_rd_zero_leave_the_quantiser():
    q, w = _case(1, B=3, S=1)
    cs = _table(16)
    rows, rt, pre, _ = oracle.q_rope_quant(q, w, 1.0, cs, 0, 1)  # position 0: cos 1, sin 0
    ref_rows, ref_rt = oracle.fp4_quant_rows(q)
    assert np.array_equal(pre, q)
    assert np.array_equal(rows, ref_rows) and np.array_equal(rt, ref_rt)
    rows0, _, pre0, _ = oracle.q_rope_quant(q, w, 1.0, np.zeros((16, 0, 2), np.float32), 7, 1,
                                            rd=0)
    assert np.array_equal(pre0, q) and np.array_equal(rows0, ref_rows)


def test_rotation_matches_float64_within_bf16_rounding():
    B, S, H = 2, 6, 4
    q, w = _case(2, B, S, H)
    start = 1000
    cs = _table(start + S)
    _, _, pre, _ = oracle.q_rope_quant(q, w, 1.0, cs, start, S)
    x = bf16_to_f32(q).astype(np.float64)
    for r in range(B * S):
        c = cs[start + r % S, :, 0].astype(np.float64)
        s = cs[start + r % S, :, 1].astype(np.float64)
        for h in range(H):
            z = x[r, h, 64:].reshape(-1, 2)
            rot = (z[:, 0] + 1j * z[:, 1]) * (c + 1j * s)  # textbook complex rotation
            got = bf16_to_f32(pre[r, h, 64:]).astype(np.float64).reshape(-1, 2)
            pair = np.hypot(rot.real, rot.imag)
            assert np.all(np.abs(got[:, 0] - rot.real) <= 2.0 ** -7 * pair + 1e-30)
            assert np.all(np.abs(got[:, 1] - rot.imag) <= 2.0 ** -7 * pair + 1e-30)
            # rotation keeps every pair's norm, to rounding
            n0 = np.hypot(z[:, 0], z[:, 1])
            assert np.all(np.abs(np.hypot(got[:, 0], got[:, 1]) - n0) <= 2.0 ** -6 * n0 + 1e-30)
        assert np.array_equal(pre[r, :, :64], q[r, :, :64])  # dims before the RoPE part


def test_rows_and_round_trip_are_the_quantisers_of_the_rotated_heads():
    q, w = _case(3, B=1, S=9, H=16)
    cs = _table(300)
    rows, rt, pre, _ = oracle.q_rope_quant(q, w, 1.0, cs, 290, 9)
    ref_rows, ref_rt = oracle.fp4_quant_rows(pre)
    assert np.array_equal(rows, ref_rows) and np.array_equal(rt, ref_rt)
    # the round trip re-quantises to the same values (what the score takes
    # as q): a block whose largest code is 3 comes back one exponent lower
    # with doubled codes, the same values in other bytes
    again, rt2 = oracle.fp4_quant_rows(rt)
    assert np.array_equal(rt2, rt)
    assert not np.array_equal(again, rows)  # this seed has such blocks


def test_weight_scaling():
    q, w = _case(4, B=2, S=3, H=64)
    cs = _table(8)
    # a power-of-two scale is exact
    _, _, _, w2 = oracle.q_rope_quant(q, w, 0.25, cs, 0, 3)
    assert np.array_equal(bf16_to_f32(w2), bf16_to_f32(w) * np.float32(0.25))
    _, _, _, w1 = oracle.q_rope_quant(q, w, 1.0, cs, 0, 3)
    assert np.array_equal(w1, w)
    # the model's scale, 128^-0.5 * 64^-0.5: within one bf16 ulp of the exact product
    sc = np.float32(128 ** -0.5 * 64 ** -0.5)
    _, _, _, ws = oracle.q_rope_quant(q, w, sc, cs, 0, 3)
    exact = bf16_to_f32(w).astype(np.float64) * float(sc)
    got = bf16_to_f32(ws).astype(np.float64)
    assert np.all(np.abs(got - exact) <= 2.0 ** -8 * np.abs(exact) + 1e-38)
    assert np.array_equal(np.signbit(got), np.signbit(exact))
    # a bf16 value times 1.5 (exact in fp32) that falls between two bf16
    # values rounds to the even one: 1 + 2^-7 is 0x3F81, times 1.5 is
    # 1.5 + 1.5 * 2^-7 = 0x3FC1 + half an ulp -> 0x3FC2 (even)
    one = np.array([[0x3F81]], np.uint16)
    _, _, _, wt = oracle.q_rope_quant(q[:1, :1], one, 1.5, cs, 0, 1)
    assert wt[0, 0] == 0x3FC2 and bf16_bits(np.float32(1.5 + 1.5 * 2.0 ** -7)) == 0x3FC2
