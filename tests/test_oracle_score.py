"""Pins of the oracle's scoring (exact dot, fixed-order head sum, masks).

Score definition: "DeepSeek V4.1" page, class Indexer, forward (the einsum
of fp4 q against index_k, relu, weights, sum over heads, compress_lens mask,
level-two candidate mask).
"""
import math
import os

import numpy as np

import oracle
from sparse_attention_top_fp4_amd.inputs import bf16_bits, bf16_to_f32, small_case

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _kcache(k_bf16):
    rows, rt = oracle.fp4_quant_rows(k_bf16)
    return rows, rt


def test_head_dots_equal_float64_matmul_of_dequantised_rows():
    c = small_case(11, B=2, S=3, H=5, T=77, start_pos=0)
    kc, krt = _kcache(c["k"])
    _, qrt = oracle.fp4_quant_rows(c["q"])
    d, inexact = oracle.head_dots(c["q"], kc, B=2, S=3, H=5, T=77)
    assert inexact == 0
    qf = bf16_to_f32(qrt).astype(np.float64)  # [R][H][128]
    kf = bf16_to_f32(krt).astype(np.float64)  # [B][T][128]
    for r in range(6):
        ref = qf[r] @ kf[r // 3].T  # exact in float64 for these magnitudes
        assert np.array_equal(d[r], ref.astype(np.float32))


def test_dot_flags_inexact_rounding():
    # block 0 at scale 2^20 and block 1 at scale 2^-20: the exact dot needs
    # more than 24 significant bits
    q = np.zeros((1, 1, 128), np.uint16)
    k = np.zeros((1, 1, 128), np.uint16)
    one = bf16_bits(np.array([1.0], np.float32))[0]
    q[0, 0, 0] = bf16_bits(np.array([2.0 ** 20], np.float32))[0]
    q[0, 0, 32] = bf16_bits(np.array([2.0 ** -20], np.float32))[0]
    k[0, 0, 0] = one
    k[0, 0, 32] = one
    kc, _ = _kcache(k)
    d, inexact = oracle.head_dots(q, kc, B=1, S=1, H=1, T=1)
    assert inexact == 1
    assert d[0, 0, 0] == np.float32(2.0 ** 20 + 2.0 ** -20)


def test_single_head_unit_weight_is_relu_of_dot():
    c = small_case(12, B=1, S=4, H=1, T=300, start_pos=0)
    kc, _ = _kcache(c["k"])
    w = bf16_bits(np.ones((4, 1), np.float32))
    cl = np.full(4, 300, np.int32)
    s, inexact = oracle.score(c["q"], w, kc, B=1, S=4, H=1, T=300, cl=cl)
    d, _ = oracle.head_dots(c["q"], kc, B=1, S=4, H=1, T=300)
    assert inexact == 0
    assert np.array_equal(s, np.maximum(d[:, 0, :], 0.0))
    assert not np.any(np.signbit(s))  # canonical +0


def _load_head_order():
    dw, expect = [], None
    for line in open(os.path.join(GOLDEN, "head_order.txt")):
        line = line.split("#")[0].strip()
        if not line:
            continue
        if line.startswith("="):
            expect = float(line[1:])
        else:
            a, b = line.split()
            dw.append((float(a), float(b)))
    return dw, expect


def test_fixed_head_order_golden():
    dw, expect = _load_head_order()
    H = len(dw)
    q = np.zeros((1, H, 128), np.uint16)
    k = np.zeros((1, 1, 128), np.uint16)
    k[0, 0, 0] = bf16_bits(np.array([1.0], np.float32))[0]
    for h, (dv, _) in enumerate(dw):
        q[0, h, 0] = bf16_bits(np.array([dv], np.float32))[0]
    w = bf16_bits(np.array([[b for _, b in dw]], np.float32))
    kc, _ = _kcache(k)
    s, inexact = oracle.score(q, w, kc, B=1, S=1, H=H, T=1, cl=np.array([1], np.int32))
    assert inexact == 0
    assert s[0, 0] == expect and not np.signbit(s[0, 0])


def test_negative_dots_contribute_nothing_and_weights_scale_exactly():
    c = small_case(13, B=1, S=2, H=64, T=64, start_pos=0)
    kc, _ = _kcache(c["k"])
    cl = np.full(2, 64, np.int32)
    s1, _ = oracle.score(c["q"], c["w"], kc, 1, 2, 64, 64, cl)
    w2 = bf16_bits(bf16_to_f32(c["w"]) * np.float32(2.0))
    s2, _ = oracle.score(c["q"], w2, kc, 1, 2, 64, 64, cl)
    assert np.array_equal(s2, s1 * np.float32(2.0))
    wz = np.zeros_like(c["w"])
    s0, _ = oracle.score(c["q"], wz, kc, 1, 2, 64, 64, cl)
    assert np.all(s0 == 0.0) and not np.any(np.signbit(s0))


def test_score_within_fma_chain_error_bound_of_exact_sum():
    c = small_case(14, B=2, S=1, H=64, T=200)
    kc, _ = _kcache(c["k"])
    s, inexact = oracle.score(c["q"], c["w"], kc, 2, 1, 64, 200, c["cl"])
    d, _ = oracle.head_dots(c["q"], kc, 2, 1, 64, 200)
    w = bf16_to_f32(c["w"]).astype(np.float64)
    u = 2.0 ** -24
    for r in range(2):
        for t in range(0, 200, 7):
            terms = [max(float(d[r, h, t]), 0.0) * float(w[r, h]) for h in range(64)]
            exact = math.fsum(terms)
            bound = 64 * u * sum(abs(x) for x in terms) + 1e-30
            assert abs(float(s[r, t]) - exact) <= bound


def test_head_permutation_changes_only_low_bits():
    """The head sum depends on its order only through rounding."""
    c = small_case(15, B=1, S=1, H=64, T=128)
    kc, _ = _kcache(c["k"])
    s, _ = oracle.score(c["q"], c["w"], kc, 1, 1, 64, 128, c["cl"])
    perm = np.random.default_rng(0).permutation(64)
    sp, _ = oracle.score(c["q"][:, perm], c["w"][:, perm], kc, 1, 1, 64, 128, c["cl"])
    d, _ = oracle.head_dots(c["q"], kc, 1, 1, 64, 128)
    mag = (np.maximum(d[0], 0) * np.abs(bf16_to_f32(c["w"][0]))[:, None]).sum(axis=0)
    assert np.all(np.abs(sp[0] - s[0]) <= 2 * 64 * 2.0 ** -24 * mag + 1e-30)


def test_causal_and_candidate_masks():
    B, S, H, T, cbs = 2, 5, 8, 96, 16
    c = small_case(16, B=B, S=S, H=H, T=T, start_pos=300, ratio=4)
    kc, _ = _kcache(c["k"])
    cl = c["cl"]
    assert list(cl[:S]) == [(300 + s + 1) // 4 for s in range(S)]
    full, _ = oracle.score(c["q"], c["w"], kc, B, S, H, T, np.full(B * S, T, np.int32))
    s, _ = oracle.score(c["q"], c["w"], kc, B, S, H, T, cl)
    t = np.arange(T)
    for r in range(B * S):
        assert np.all(np.isneginf(s[r, t >= cl[r]]))
        assert np.array_equal(s[r, t < cl[r]], full[r, t < cl[r]])
    cand = np.array([[0, 2, 5]] * (B * S), np.int32)
    sc, _ = oracle.score(c["q"], c["w"], kc, B, S, H, T, cl, cand=cand, cbs=cbs)
    inblk = np.isin(t // cbs, [0, 2, 5])
    for r in range(B * S):
        keep = (t < cl[r]) & inblk
        assert np.array_equal(sc[r, keep], full[r, keep])
        assert np.all(np.isneginf(sc[r, ~keep]))
    # every block a candidate == no candidate mask
    allc = np.tile(np.arange(T // cbs, dtype=np.int32), (B * S, 1))
    sa, _ = oracle.score(c["q"], c["w"], kc, B, S, H, T, cl, cand=allc, cbs=cbs)
    assert np.array_equal(sa, s)
