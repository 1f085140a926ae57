"""CPU oracle for the DeepSeek-V4.1 Indexer hot path -- TEST INFRASTRUCTURE.

Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product path (the HIP library and
its Python binding) never imports, links or calls anything here, and this
package imports nothing from the product.

The arithmetic lives in ``oracle.c`` (plain C, OpenMP over rows, built with
``-O2 -ffp-contract=off``); this module builds it with gcc when needed and
marshals numpy arrays through ctypes.  ``topk_bruteforce`` and
``select_blocks_bruteforce`` below are independent pure-numpy restatements
used to pin the C code on tiny inputs.

Pages cited (by page and section):
  [IDX]  "DeepSeek V4.1" -- class Indexer (atlas.klimoza.dev, .../indexer/index-keys)
  [CMP]  "Module compress" -- Rust CPU reference API (docs.atlascybernetics.ai)
  [VLLM] "launcher/.../patches/attention.py" -- vLLM DeepseekV4 patch (git.kilork.org)

Parity status per function (what pins it; see tests/test_oracle_*.py):
  fp4_quant_rows   pinned: exhaustive e8m0 exponent vs exact rationals, e2m1
                   tie table, nearest-point property, idempotence.
  head_dots        pinned: equals float64 matmul of the dequantised rows.
  score            pinned: H=1 reduces to relu(d); a hand-worked order case;
                   fsum error bound; masks by brute force.
  topk             pinned: numpy lexsort brute force; width/order/-1 invariants;
                   the short-context closed form [VLLM, _fill_short_context_topk_indices].
  select_blocks    pinned: numpy brute force; ctb >= nb keeps every reachable block.
  yarn_cos_sin     float64 numpy, written here (not in oracle.c).  Pinned:
                   factor 1 is plain RoPE; the correction dimension of beta
                   rotations satisfies its defining equation; the band
                   (lo, hi) = (20, 33) hand-worked for the chosen constants;
                   hand-worked frequency ratios inside the band.  The
                   constants themselves are a reading (the pages name them
                   only).
  fp8_quant_rows   pinned: the e4m3 value table against the format's
                   definition, exhaustive ue8m0 exponent vs exact rationals,
                   a hand-worked tie table (tests/golden/e4m3_rne_ties.txt),
                   the nearest-point property over all bf16, idempotence.
  head_dots_fp8    pinned: the float64 matmul of the dequantised rows,
                   rounded once to fp32.
  score_fp8        pinned: on fp4 round trips with equal block scales (exactly
                   representable in e4m3) it equals score() bit for bit.
  score_bf16_literal  DIAGNOSTIC only (not compared with the GPU): the page's
                   bf16 tensor pipeline, for the top-k overlap against the
                   fp32 contract.  Pinned: one head with unit weight gives
                   bf16(relu(dot)); the fp4 row decoding equals the
                   quantiser's round trip.
  head sum order   the fp32 two-chain association is a contract shared with
                   the GPU library (split chosen to match the matrix core's
                   half-wave layout); the pages fix none.  A hand-worked
                   golden tells it apart from the other plausible orders.
  publish          pinned: pre-quantisation key vs a float64 restatement within
                   bf16 rounding; RoPE identity at position 0; norm preservation.
  topk_pairs,      the T-split top-k, numpy over topk().  Pinned: merging the
  merge_topk       slices' lists equals topk() of the whole row for every
                   slicing tried (ties across slice edges, -0 and +0,
                   compress_lens in every slice, k beyond a slice's width);
                   a hand-worked two-slice tie; the full-lexsort brute force
                   on tiny rows.
  q_rope_quant     pinned: RoPE identity at position 0 and with rd = 0 (the
                   rows are then the quantiser's); rotation vs a float64
                   restatement within bf16 rounding; pair norms; weights
                   exact for power-of-two scales, within one bf16 ulp of the
                   float64 product otherwise; the round trip re-quantises to
                   the same rows.
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

_lib = None


def build(force: bool = False) -> str:
    """Compile oracle.c into liboracle.so with gcc."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        cmd = ["gcc", "-std=c11", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
               "-fPIC", "-shared", "-D_GNU_SOURCE", _SRC, "-o", _LIB + ".tmp", "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(_LIB + ".tmp", _LIB)
    return _LIB


def lib():
    global _lib
    if _lib is None:
        build()
        L = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        i64, i32, f32, f64 = ctypes.c_int64, ctypes.c_int, ctypes.c_float, ctypes.c_double
        L.orc_fp4_quant_rows.argtypes = [P, i64, P, P]
        L.orc_fp4_quant_rows.restype = None
        L.orc_head_dots.argtypes = [P, P, i64, i32, i32, i32, i32, P]
        L.orc_head_dots.restype = i64
        L.orc_score.argtypes = [P, P, P, i64, i32, i32, i32, i32, P, P, i32, i32, P, i64]
        L.orc_score.restype = i64
        L.orc_topk.argtypes = [P, i64, i32, i32, P, i32, ctypes.c_int32, P, i64]
        L.orc_topk.restype = None
        L.orc_select_blocks.argtypes = [P, i64, i32, i32, P, i32, i32, P, i64]
        L.orc_select_blocks.restype = None
        L.orc_publish.argtypes = [P, P, P, P, i32, i32, i32, i32, i32, f32, i32, i32, P, i64, P]
        L.orc_q_rope_quant.argtypes = [P, P, f32, P, i32, i32, i32, i32, i32, i32, P, P, P, P]
        L.orc_q_rope_quant.restype = None
        L.orc_publish.restype = None
        L.orc_fp8_quant_rows.argtypes = [P, i64, P, P]
        L.orc_fp8_quant_rows.restype = None
        L.orc_head_dots_fp8.argtypes = [P, P, i64, i32, i32, i32, i32, P]
        L.orc_head_dots_fp8.restype = i64
        L.orc_score_fp8.argtypes = [P, P, P, i64, i32, i32, i32, i32, P, P, i32, i32, P, i64]
        L.orc_score_fp8.restype = i64
        _lib = L
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    a = np.ascontiguousarray(a, dtype=dtype)
    return a


# ----------------------------------------------------------------- quantiser
def fp4_quant_rows(x_bf16: np.ndarray):
    """[IDX, forward: fp4_act_quant]; [CMP, fp4_quant_e8m0_inplace].

    x_bf16: uint16 [..., 128] bf16 bit patterns.  Returns (rows uint8
    [..., 68], roundtrip uint16 [..., 128])."""
    x = _c(x_bf16, np.uint16)
    assert x.shape[-1] == 128
    n = x.size // 128
    rows = np.empty(x.shape[:-1] + (68,), np.uint8)
    rt = np.empty_like(x)
    lib().orc_fp4_quant_rows(_p(x), n, _p(rows), _p(rt))
    return rows, rt


# ---------------------------------------------------------------- scoring
def head_dots(q, kc, B, S, H, T):
    """Exact per-head dots d[r][h][t] (fp32).  q uint16 [R][H][128], kc uint8
    [B][Tcap][68].  Returns (d, inexact_count)."""
    q = _c(q, np.uint16)
    kc = _c(kc, np.uint8)
    kstride = kc.shape[1]
    d = np.empty((B * S, H, T), np.float32)
    inexact = lib().orc_head_dots(_p(q), _p(kc), kstride, B, S, H, T, _p(d))
    return d, inexact


def score(q, w, kc, B, S, H, T, cl, cand=None, cbs=0):
    """[IDX, forward: index_score with relu, weights, head sum, masks].

    Returns (scores float32 [R][T] with every t < T defined, inexact_count)."""
    q = _c(q, np.uint16)
    w = _c(w, np.uint16)
    kc = _c(kc, np.uint8)
    cl = _c(cl, np.int32)
    R = B * S
    assert q.shape[:2] == (R, H) and w.shape == (R, H) and cl.shape == (R,) and H <= 1024
    kstride = kc.shape[1]
    n_cand = 0
    if cand is not None:
        cand = _c(cand, np.int32)
        n_cand = cand.shape[1]
    out = np.empty((R, T), np.float32)
    inexact = lib().orc_score(_p(q), _p(w), _p(kc), kstride, B, S, H, T, _p(cl), _p(cand),
                              n_cand, cbs, _p(out), T)
    return out, inexact


# ------------------------------------------------------------ FP8 cache
def fp8_quant_rows(x_bf16: np.ndarray):
    """[VLLM, _indexer_k_cache_head_dim] FP8 rows: e4m3 codes with one ue8m0
    scale (stored fp32) per 128 values.  x_bf16: uint16 [..., 128].  Returns
    (rows uint8 [..., 132], roundtrip uint16 [..., 128])."""
    x = _c(x_bf16, np.uint16)
    assert x.shape[-1] == 128
    n = x.size // 128
    rows = np.empty(x.shape[:-1] + (132,), np.uint8)
    rt = np.empty_like(x)
    lib().orc_fp8_quant_rows(_p(x), n, _p(rows), _p(rt))
    return rows, rt


def head_dots_fp8(q, kc, B, S, H, T):
    """Per-head dots on FP8 rows, each the exact sum rounded once to fp32.
    kc uint8 [B][Tcap][132].  Returns (d, count of dots rounded)."""
    q = _c(q, np.uint16)
    kc = _c(kc, np.uint8)
    d = np.empty((B * S, H, T), np.float32)
    n = lib().orc_head_dots_fp8(_p(q), _p(kc), kc.shape[1], B, S, H, T, _p(d))
    return d, n


def score_fp8(q, w, kc, B, S, H, T, cl, cand=None, cbs=0):
    """score() on the FP8 cache (kc uint8 [B][Tcap][132]); q is quantised
    per head by the FP8 quantiser.  Returns (scores, count of dots rounded)."""
    q = _c(q, np.uint16)
    w = _c(w, np.uint16)
    kc = _c(kc, np.uint8)
    cl = _c(cl, np.int32)
    R = B * S
    assert q.shape[:2] == (R, H) and w.shape == (R, H) and cl.shape == (R,) and H <= 1024
    n_cand = 0
    if cand is not None:
        cand = _c(cand, np.int32)
        n_cand = cand.shape[1]
    out = np.empty((R, T), np.float32)
    n = lib().orc_score_fp8(_p(q), _p(w), _p(kc), kc.shape[1], B, S, H, T, _p(cl), _p(cand),
                            n_cand, cbs, _p(out), T)
    return out, n


# ------------------------------------------------------------------- top-k
def topk(scores, cl, k, offset=0, T=None):
    """[IDX, forward: top-k, position re-sort, -1 and offset]."""
    scores = _c(scores, np.float32)
    cl = _c(cl, np.int32)
    R = scores.shape[0]
    T = scores.shape[1] if T is None else T
    kout = min(k, T)
    out = np.empty((R, kout), np.int32)
    lib().orc_topk(_p(scores), scores.shape[1], R, T, _p(cl), k, offset, _p(out), kout)
    return out


def select_blocks(scores, cl, ctb, cbs, T=None):
    """[IDX, forward: select_candidate_blocks] (body not on the pages; block
    max reading)."""
    scores = _c(scores, np.float32)
    cl = _c(cl, np.int32)
    R = scores.shape[0]
    T = scores.shape[1] if T is None else T
    nb = (T + cbs - 1) // cbs
    kk = min(ctb, nb)
    ids = np.empty((R, kk), np.int32)
    lib().orc_select_blocks(_p(scores), scores.shape[1], R, T, _p(cl), ctb, cbs, _p(ids), kk)
    return ids


# ---------------------------------------------------------------- publish
def yarn_correction_dim(beta, rd, theta, orig_len):
    """[CMP, yarn_freqs_cis] (YaRN, Peng et al., the "NTK-by-parts" band):
    dimension pair i of a rd-wide RoPE turns orig_len * theta^(-2i/rd) /
    (2 pi) times over the original context.  The correction dimension of
    beta rotations is the real d at which that count equals beta, i.e. the
    solution of theta^(2d/rd) = orig_len / (2 pi beta), found here as a
    logarithm to base theta."""
    return 0.5 * rd * math.log(orig_len / (2.0 * math.pi * beta), theta)


def yarn_correction_range(rd, theta, orig_len, beta_fast, beta_slow):
    """The integer band [lo, hi] of the ramp: lo = floor(d(beta_fast)) and
    hi = ceil(d(beta_slow)), kept inside [0, rd - 1] (the clamp of
    precompute_freqs_cis, which the page names as the table's builder)."""
    lo = math.floor(yarn_correction_dim(beta_fast, rd, theta, orig_len))
    hi = math.ceil(yarn_correction_dim(beta_slow, rd, theta, orig_len))
    return max(lo, 0), min(hi, rd - 1)


def yarn_frequencies(rd, theta, factor, orig_len, beta_fast, beta_slow):
    """Rotation frequency of each of the rd/2 dimension pairs, float64.
    Plain RoPE: theta^(-2i/rd).  With YaRN (orig_len > 0, factor != 1) pair
    i moves from the plain frequency (below the band) to the plain frequency
    divided by factor (above it) along a straight line in i across the band
    (a band of width 0 is widened to 0.001)."""
    i = np.arange(rd // 2, dtype=np.float64)
    plain = np.power(float(theta), -2.0 * i / rd)
    if orig_len <= 0 or factor == 1.0:
        return plain
    lo, hi = yarn_correction_range(rd, theta, orig_len, beta_fast, beta_slow)
    width = float(hi - lo) if hi != lo else 0.001
    ramp = np.clip((i - lo) / width, 0.0, 1.0)  # 0: plain, 1: plain / factor
    return plain * (1.0 - ramp) + (plain / factor) * ramp


def yarn_cos_sin(P, rd, theta, factor, orig_len, beta_fast, beta_slow):
    """[CMP, yarn_freqs_cis]: the [P][rd/2] table of (cos, sin) of position p
    times each pair's frequency, in float64, stored float32 ([P, rd/2, 2]).
    Built in row chunks to bound memory for long tables."""
    f = yarn_frequencies(rd, theta, factor, orig_len, beta_fast, beta_slow)
    out = np.empty((P, rd // 2, 2), np.float32)
    for p0 in range(0, P, 1 << 16):
        pos = np.arange(p0, min(P, p0 + (1 << 16)), dtype=np.float64)
        ang = pos[:, None] * f[None, :]
        out[p0:p0 + len(pos), :, 0] = np.cos(ang)
        out[p0:p0 + len(pos), :, 1] = np.sin(ang)
    return out


def publish(latent, wk, gamma, cos_sin, start_pos, ratio, eps, kc, rd=64):
    """[IDX, forward: index-key publish].  latent uint16 [B][G][Din], wk
    uint16 [128][Din], gamma float32 [128], cos_sin float32 [P][rd/2][2],
    kc uint8 [B][Tcap][68] updated in place.  Returns the pre-quantisation
    keys uint16 [B][G][128]."""
    latent = _c(latent, np.uint16)
    wk = _c(wk, np.uint16)
    gamma = _c(gamma, np.float32)
    cos_sin = _c(cos_sin, np.float32)
    assert kc.flags.c_contiguous and kc.dtype == np.uint8
    B, G, Din = latent.shape
    pre = np.empty((B, G, 128), np.uint16)
    lib().orc_publish(_p(latent), _p(wk), _p(gamma), _p(cos_sin), cos_sin.shape[0], B, G, Din, rd,
                      eps, start_pos, ratio, _p(kc), kc.shape[1], _p(pre))
    return pre


def q_rope_quant(q, w_raw, scale, cos_sin, start_pos, S, rd=64):
    """[IDX, forward: RoPE on the query heads' last rd dims at positions
    start_pos + s, fp4_act_quant, weights_proj(x) * scale];
    [VLLM, fused_indexer_q_rope_quant].  q uint16 [B*S][H][128] (before
    RoPE), w_raw uint16 [B*S][H], scale float32, cos_sin float32
    [P][rd/2][2].  Returns (rows uint8 [B*S][H][68], round trip uint16
    [B*S][H][128], pre-quantisation uint16 [B*S][H][128], weights uint16
    [B*S][H])."""
    q = _c(q, np.uint16)
    w_raw = _c(w_raw, np.uint16)
    cos_sin = _c(cos_sin, np.float32)
    R, H, _ = q.shape
    assert R % S == 0 and w_raw.shape == (R, H)
    rows = np.empty((R, H, 68), np.uint8)
    rt = np.empty((R, H, 128), np.uint16)
    pre = np.empty((R, H, 128), np.uint16)
    w_out = np.empty((R, H), np.uint16)
    lib().orc_q_rope_quant(_p(q), _p(w_raw), float(np.float32(scale)), _p(cos_sin),
                           cos_sin.shape[0], R // S, S, H, rd, start_pos, _p(rows), _p(rt),
                           _p(pre), _p(w_out))
    return rows, rt, pre, w_out


# ------------------------------------------- literal bf16 pipeline (C6)
def _bf16_round(x):
    """float64 -> nearest bf16 value (ties to even), as float64, through
    float32 (exact for the values used here: every input is a float32)."""
    f = np.ascontiguousarray(x, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
    return r.astype(np.uint32).view(np.float32).astype(np.float64)


def score_bf16_literal(q, w, kc, S, H, T, cl):
    """DIAGNOSTIC, not the contract: the Indexer's score as the page's torch
    ops compute it in bf16 ([IDX, forward]: einsum of the fp4 round trips
    into a bf16 tensor, relu_, times weights.unsqueeze(-1) into bf16,
    .sum(dim=2) into bf16; [CMP] 'Module compress', precision: the scores
    are bf16 tensors).  The einsum's dots are exact in fp32 (so bf16 of the
    exact dot), the elementwise product is rounded to bf16, and the head sum
    is accumulated in float64 and rounded once to bf16 (a bf16 reduction
    accumulates wider than bf16; its order is the library's).  Positions
    t >= cl are -inf.  Returns float64 [R][T]."""
    _, qrt = fp4_quant_rows(q)
    kd = np.stack([_dequant_rows(kc[b, :T]) for b in range(kc.shape[0])])
    qd = (np.ascontiguousarray(qrt, np.uint16).astype(np.uint32) << 16).view(np.float32)
    wd = (np.ascontiguousarray(w, np.uint16).astype(np.uint32) << 16).view(np.float32)
    R = q.shape[0]
    out = np.full((R, T), -np.inf)
    for r in range(R):
        d = qd[r].astype(np.float64) @ kd[r // S].T.astype(np.float64)   # [H][T], exact
        e = _bf16_round(np.maximum(_bf16_round(d), 0.0))                  # einsum, relu_
        m = _bf16_round(e * wd[r][:, None].astype(np.float64))            # * weights
        sc = _bf16_round(m.sum(axis=0))                                   # sum over heads
        c = int(min(max(cl[r], 0), T))
        out[r, :c] = sc[:c]
    return out


def _dequant_rows(rows68):
    """fp4 rows [n][68] -> their values [n][128] float32 (decoding the row
    layout: element 2i in the low nibble of byte i, byte 64+j = e_j + 127)."""
    rows68 = np.ascontiguousarray(rows68, np.uint8)
    nib = np.empty(rows68.shape[:-1] + (128,), np.uint8)
    nib[..., 0::2] = rows68[..., :64] & 0xF
    nib[..., 1::2] = rows68[..., :64] >> 4
    grid = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6], np.float64)
    mag = grid[nib & 7]
    sgn = np.where(nib & 8, -1.0, 1.0)
    e = rows68[..., 64:68].astype(np.int64) - 127
    scale = np.ldexp(1.0, np.repeat(e, 32, axis=-1))
    return (sgn * mag * scale).astype(np.float32)


def topk_overlap(s_a, s_b, cl, k):
    """Mean over rows of |top-k(s_a) & top-k(s_b)| / k_row (ties to the lower
    position on both sides)."""
    a = topk(np.asarray(s_a, np.float32), cl, k)
    b = topk(np.asarray(s_b, np.float32), cl, k)
    fr = []
    for r in range(a.shape[0]):
        ra, rb = set(a[r][a[r] >= 0].tolist()), set(b[r][b[r] >= 0].tolist())
        fr.append(len(ra & rb) / max(1, len(ra)))
    return float(np.mean(fr))


# ------------------------------------------------- tiny numpy brute force
def topk_bruteforce(scores_row: np.ndarray, cl: int, k: int, offset: int = 0) -> np.ndarray:
    """Independent restatement for tiny rows: a full lexsort by (-score, t)."""
    T = scores_row.shape[0]
    t = np.arange(T)
    s = np.where(t < cl, scores_row.astype(np.float64), -np.inf)
    s = np.where(s == 0.0, 0.0, s)  # -0 ties with +0
    order = np.lexsort((t, -s))[: min(k, T)]
    order = np.sort(order)
    return np.where(order < cl, order + offset, -1).astype(np.int32)


def topk_pairs(scores, cl, k, start, T_slice):
    """The top-k of the slice [start, start + T_slice) of each row as pairs
    ([IDX, forward: topk of the masked scores, position re-sort, -1 where not
    below compress_lens]; the T-split of a row over several owners): the
    slice ranked by topk() with compress_lens clamp(cl - start, 0, T_slice)
    and offset start, so the positions are the row's; and the score of each
    listed position, -inf for -1.  Returns (pos [R][k_out] int32, score
    [R][k_out] float32), k_out = min(k, T_slice)."""
    scores = np.asarray(scores, np.float32)
    sl = np.ascontiguousarray(scores[:, start:start + T_slice])
    lens = np.clip(np.asarray(cl, np.int64) - start, 0, T_slice).astype(np.int32)
    pos = topk(sl, lens, k, offset=start)
    idx = np.clip(pos.astype(np.int64) - start, 0, max(T_slice - 1, 0))
    got = np.take_along_axis(sl, idx, axis=1) if T_slice else np.zeros_like(pos, np.float32)
    sc = np.where(pos >= 0, got, np.float32(-np.inf)).astype(np.float32)
    return pos, sc


def merge_topk(pos, score, cl, T, k, offset=0):
    """The rows' top-k from their slices' pairs (pos, score [G][R][n], list g
    of row r from slice g, -1 entries skipped).  A position in the row's top
    k is beaten by fewer than k positions of the row, hence of its slice, so
    the union of the slices' lists holds it; the union is ranked here by a
    full sort on (score descending, -0 equal to +0; position ascending), the
    first k_out = min(k, T) kept and written by position as position +
    offset (-1 at or past compress_lens).  Rows with compress_lens <= k_out
    take the closed form; with fewer valid pairs than k_out, every valid pair
    is written and the rest is -1."""
    pos = np.asarray(pos, np.int32)
    score = np.asarray(score, np.float32)
    G, R, n = pos.shape
    kout = min(k, T)
    out = np.full((R, kout), -1, np.int32)
    ar = np.arange(kout)
    for r in range(R):
        c = min(max(int(cl[r]), 0), T)
        if c <= kout:
            out[r] = np.where(ar < c, ar + offset, -1)
            continue
        p = pos[:, r, :].reshape(-1).astype(np.int64)
        s = score[:, r, :].reshape(-1).astype(np.float64)
        keep = p >= 0
        p, s = p[keep], s[keep]
        s = np.where(s == 0.0, 0.0, s)
        sel = np.sort(p[np.lexsort((p, -s))[:kout]])
        out[r, :sel.size] = np.where(sel < c, sel + offset, -1)
    return out


def select_blocks_bruteforce(scores_row, cl, ctb, cbs):
    T = scores_row.shape[0]
    c = min(cl, T)
    nb = (T + cbs - 1) // cbs
    s = np.where(np.arange(T) < c, scores_row.astype(np.float64), -np.inf)
    bm = np.array([s[j * cbs: min((j + 1) * cbs, T)].max() for j in range(nb)])
    return topk_bruteforce(bm, (c + cbs - 1) // cbs, ctb, 0)
