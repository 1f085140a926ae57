"""The C ABI library on the host: it loads, exports every entry point that
include/idx.h declares, rejects invalid arguments before launching anything,
and its host-side RoPE table agrees with the oracle's.  No GPU needed."""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle
import sparse_attention_top_fp4_amd as idx
from sparse_attention_top_fp4_amd.inputs import YARN

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
IDX_OK, IDX_EINVAL, IDX_EUNSUPPORTED = 0, 1, 2


def _declared_symbols():
    """Every idx_* function declared in include/*.h."""
    syms = set()
    for name in sorted(os.listdir(os.path.join(ROOT, "include"))):
        if name.endswith(".h"):
            text = open(os.path.join(ROOT, "include", name)).read()
            text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
            syms |= set(re.findall(r"\b(idx_[a-z0-9_]+)\s*\(", text))
    return sorted(syms)


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(idx.library_path()):
        from sparse_attention_top_fp4_amd import build
        build.build()
    return idx.load_library()


def test_exports_every_declared_symbol(lib):
    syms = _declared_symbols()
    assert len(syms) >= 9
    for s in syms:
        assert hasattr(lib, s), s


def test_status_strings(lib):
    for code in range(4):
        assert lib.idx_status_string(code).startswith(b"IDX_")


def test_score_rejects_bad_arguments_without_launching(lib):
    P = ctypes.c_void_p
    dummy = P(0x1000)  # never dereferenced: validation fails first
    # D != 128 and unsupported head counts
    assert lib.idx_score(dummy, dummy, dummy, 8, 1, 1, 64, 64, 8, dummy, None, 0, 0, dummy, 8,
                         None, None) == IDX_EUNSUPPORTED
    assert lib.idx_score(dummy, dummy, dummy, 8, 1, 1, 48, 128, 8, dummy, None, 0, 0, dummy, 8,
                         None, None) == IDX_EUNSUPPORTED
    # null pointers, short row stride, short cache stride, bad candidates
    assert lib.idx_score(None, dummy, dummy, 8, 1, 1, 64, 128, 8, dummy, None, 0, 0, dummy, 8,
                         None, None) == IDX_EINVAL
    assert lib.idx_score(dummy, dummy, dummy, 8, 1, 1, 64, 128, 8, dummy, None, 0, 0, dummy, 7,
                         None, None) == IDX_EINVAL
    assert lib.idx_score(dummy, dummy, dummy, 7, 1, 1, 64, 128, 8, dummy, None, 0, 0, dummy, 8,
                         None, None) == IDX_EINVAL
    assert lib.idx_score(dummy, dummy, dummy, 8, 1, 1, 64, 128, 8, dummy, dummy, 0, 128, dummy, 8,
                         None, None) == IDX_EINVAL
    assert lib.idx_score(dummy, dummy, dummy, 8, -1, 1, 64, 128, 8, dummy, None, 0, 0, dummy, 8,
                         None, None) == IDX_EINVAL
    # empty work is a no-op, even with null pointers
    assert lib.idx_score(None, None, None, 0, 0, 1, 64, 128, 8, None, None, 0, 0, None, 8,
                         None, None) == IDX_OK


def test_topk_and_select_reject_bad_arguments(lib):
    P = ctypes.c_void_p
    d = P(0x1000)
    assert lib.idx_topk(d, 8, 1, 8, d, None, 0, 0, d, 8, None, None, 0, None) == IDX_EINVAL  # topk 0
    assert lib.idx_topk(d, 7, 1, 8, d, None, 4, 0, d, 8, None, None, 0, None) == IDX_EINVAL  # ld < T
    assert lib.idx_topk(d, 8, 1, 8, d, None, 4, 0, d, 3, None, None, 0, None) == IDX_EINVAL  # ld_out < k
    assert lib.idx_topk(None, 8, 0, 8, None, None, 4, 0, None, 8, None, None, 0, None) == IDX_OK  # R = 0
    need = lib.idx_topk_workspace_size(4, 100000, 2048)
    assert need > 0
    assert lib.idx_topk(d, 100000, 4, 100000, d, None, 2048, 0, d, 2048, None, None, 0, None) == IDX_EINVAL
    assert lib.idx_select_candidate_blocks(d, 8, 1, 8, d, 0, 4, d, 2, None, 0, None) == IDX_EINVAL
    assert lib.idx_select_candidate_blocks(d, 8, 1, 8, d, 2, 4, d, 1, d, 1 << 20,
                                           None, None) == IDX_EINVAL  # ld_ids < min(ctb, nb)
    assert lib.idx_topk_workspace_size(4, 512, 2048) == 0  # every position kept


def test_publish_rejects_bad_arguments(lib):
    d = ctypes.c_void_p(0x1000)
    args = dict(P=100, B=1, G=1, Din=512, D=128, rd=64, eps=1e-6, sp=39, ratio=4, stride=64,
                Tcap=64)

    def call(**kw):
        a = dict(args, **kw)
        return lib.idx_publish_keys(d, d, d, d, a["P"], a["B"], a["G"], a["Din"], a["D"], a["rd"],
                                    a["eps"], a["sp"], a["ratio"], d, a["stride"], a["Tcap"], None)

    assert call(D=64) == IDX_EUNSUPPORTED
    assert call(rd=63) == IDX_EINVAL
    assert call(G=2) == IDX_EINVAL  # decode publishes one group
    assert call(P=36) == IDX_EINVAL  # position 36 not in the table
    assert call(sp=4 * 64 + 3) == IDX_EINVAL  # row 64 beyond Tcap
    assert call(sp=2) == IDX_EINVAL  # start_pos + 1 - ratio < 0
    assert call(stride=10) == IDX_EINVAL
    assert call(B=0) == IDX_OK


def test_quant_rejects_bad_arguments(lib):
    assert lib.idx_fp4_quant(None, -1, None, None, None) == IDX_EINVAL
    assert lib.idx_fp4_quant(None, 0, None, None, None) == IDX_OK
    assert lib.idx_fp4_quant(None, 3, None, None, None) == IDX_EINVAL


def test_host_rope_table_matches_oracle(lib):
    """The library's table (C, libm) against the oracle's own float64 numpy
    table, which the tests pin to hand-worked values: within one fp32 rounding
    of each other (the two float64 cosines may differ in their last bits)."""
    for factor, orig in ((YARN["factor"], YARN["orig_len"]), (1.0, 0), (4.0, 4096)):
        a = idx.idx_yarn_cos_sin(5000, 64, YARN["theta"], factor, orig, YARN["beta_fast"],
                                 YARN["beta_slow"])
        b = oracle.yarn_cos_sin(5000, 64, YARN["theta"], factor, orig, YARN["beta_fast"],
                                YARN["beta_slow"])
        diff = np.abs(a.astype(np.float64) - b.astype(np.float64))
        assert diff.max() <= 2.0 ** -24
        assert np.mean(a == b) > 0.999


def test_host_rope_table_rejects_bad_arguments(lib):
    out = (ctypes.c_float * 64)()
    assert lib.idx_yarn_cos_sin(1, 63, 1e4, 1.0, 0, 32.0, 1.0, out) == IDX_EINVAL
    assert lib.idx_yarn_cos_sin(1, 64, 1.0, 1.0, 0, 32.0, 1.0, out) == IDX_EINVAL
    assert lib.idx_yarn_cos_sin(1, 64, 1e4, 16.0, 65536, 0.0, 1.0, out) == IDX_EINVAL
    assert lib.idx_yarn_cos_sin(1, 64, 1e4, 16.0, 65536, 32.0, 1.0, None) == IDX_EINVAL
    assert lib.idx_yarn_cos_sin(0, 64, 1e4, 16.0, 65536, 32.0, 1.0, None) == IDX_OK


def test_fused_score_topk_rejects_bad_arguments(lib):
    d = ctypes.c_void_p(0x1000)
    # rows wider than one workgroup ranks
    assert lib.idx_score_topk(d, d, d, 9000, 1, 1, 64, 128, 8193, d, 2048, 0, d, 2048, None, 0,
                              None) == IDX_EUNSUPPORTED
    assert lib.idx_score_topk(d, d, d, 64, 1, 1, 64, 128, 64, d, 0, 0, d, 64, None, 0,
                              None) == IDX_EINVAL  # index_topk 0
    assert lib.idx_score_topk(d, d, d, 64, 1, 1, 64, 128, 64, d, 32, 0, d, 31, None, 0,
                              None) == IDX_EINVAL  # ld_out < k_out
    assert lib.idx_score_topk(d, d, d, 64, 1, 1, 64, 128, 64, d, 32, 0, d, 32, d, 63,
                              None) == IDX_EINVAL  # scores ld < T
    assert lib.idx_score_topk(d, d, d, 64, 1, 1, 48, 128, 64, d, 32, 0, d, 32, None, 0,
                              None) == IDX_EUNSUPPORTED  # 48 heads
    assert lib.idx_score_topk(None, None, None, 0, 0, 1, 64, 128, 64, None, 32, 0, None, 32,
                              None, 0, None) == IDX_OK  # no rows


def test_two_level_topk_checks_before_launch(lib):
    """Both levels' checks, and one histogram passed for both levels, are
    refused before anything launches."""
    d = ctypes.c_void_p(0x1000)
    h1, h2 = ctypes.c_void_p(0x2000), ctypes.c_void_p(0x3000)

    def call(B=2, T=65536, ld=65536, ld_out1=2048, hist1=h1, hist2=h2, n_cand=64, cbs=128,
             ld2=8192, k=2048, ld_out2=2048, H=64):
        return lib.idx_two_level_topk(d, ld, hist1, d, ld_out1, d, 1 << 30, d, d, d, T, B, 1, H,
                                      128, T, d, d, n_cand, cbs, d, ld2, hist2, k, 0, d, ld_out2,
                                      None)
    assert call(hist2=h1) == IDX_EINVAL        # one histogram for both levels
    assert call(ld=65535) == IDX_EINVAL        # level one: ld < T
    assert call(ld_out1=2047) == IDX_EINVAL    # level one: ld_out < k_out
    assert call(ld2=8191) == IDX_EINVAL        # level two: slot row shorter than the slots
    assert call(ld_out2=2047) == IDX_EINVAL    # level two: ld_out < k_out
    assert call(T=70000, ld=70000) == IDX_EUNSUPPORTED  # level two's rows past 65536
    assert call(n_cand=0) == IDX_EINVAL
    assert call(k=0) == IDX_EINVAL
    assert call(B=0) == IDX_OK                 # no rows


def test_score_with_query_step_checks_its_arguments(lib):
    """The query step's arguments of idx_score_qrope / idx_score_topk_qrope
    are refused before any launch, as idx_q_rope_quant refuses them."""
    d = ctypes.c_void_p(0x1000)
    f = ctypes.c_float(1.0)

    def score(rd=64, sp=10, P=20, S=4, cs=d):
        return lib.idx_score_qrope(d, d, f, cs, P, rd, sp, d, 64, 1, S, 64, 128, 64, d, d, 64,
                                   None, None)

    def topk(rd=64, sp=10, P=20, S=4, cs=d):
        return lib.idx_score_topk_qrope(d, d, f, cs, P, rd, sp, d, 64, 1, S, 64, 128, 64, d, 32, 0,
                                        d, 32, None, 0, None)
    for call in (score, topk):
        assert call(rd=63) == IDX_EINVAL          # odd rd
        assert call(rd=130) == IDX_EINVAL         # rd past the head
        assert call(sp=17, P=20) == IDX_EINVAL    # position 20 not in the table
        assert call(sp=-1) == IDX_EINVAL
        assert call(cs=None) == IDX_EINVAL        # no table with rd > 0
        assert call(cs=ctypes.c_void_p(0x1004)) == IDX_EINVAL  # table not 8-byte aligned
    assert lib.idx_score_qrope(d, d, f, None, 0, 0, 0, d, 64, 0, 1, 64, 128, 64, d, d, 64, None,
                               None) == IDX_OK   # rd 0, no rows


def test_bf16_probe_rejects_null_pointers(lib):
    n = ctypes.c_ulonglong(0)
    assert lib.idx_probe_bf16_convert(None, ctypes.byref(n), None) == IDX_EINVAL
    assert lib.idx_probe_bf16_convert(ctypes.c_void_p(0x1000), None, None) == IDX_EINVAL
    assert lib.idx_probe_bf16_convert(ctypes.c_void_p(0x1004), ctypes.byref(n), None) == IDX_EINVAL


def test_candidate_topk_rejects_bad_arguments(lib):
    d = ctypes.c_void_p(0x1000)
    assert lib.idx_topk_candidates(d, 70000, 1, 70000, d, d, 64, 128, None, 2048, 0, d, 2048,
                                   None, None) == IDX_EUNSUPPORTED  # row wider than the bit map
    assert lib.idx_topk_candidates(d, 65536, 1, 65536, d, d, 65, 128, None, 2048, 0, d, 2048,
                                   None, None) == IDX_EUNSUPPORTED  # more than 8192 candidate slots
    assert lib.idx_topk_candidates(d, 8, 1, 8, d, d, 0, 4, None, 4, 0, d, 4,
                                   None, None) == IDX_EINVAL
    assert lib.idx_topk_candidates(d, 8, 1, 8, d, d, 2, 4, None, 4, 0, d, 3,
                                   None, None) == IDX_EINVAL
    assert lib.idx_topk_candidates(None, 8, 0, 8, None, None, 2, 4, None, 4, 0, None, 4,
                                   None, None) == IDX_OK


def test_topk_reports_k_out(lib):
    """idx_topk and idx_topk_candidates write the row width min(index_topk, T)
    to the host k_out once their arguments pass (no device work here: R = 0)."""
    k = ctypes.c_int32(-1)
    assert lib.idx_topk(None, 8, 0, 8, None, None, 4, 0, None, 8, ctypes.byref(k), None, 0,
                        None) == IDX_OK and k.value == 4
    assert lib.idx_topk(None, 8, 0, 8, None, None, 20, 0, None, 8, ctypes.byref(k), None, 0,
                        None) == IDX_OK and k.value == 8
    k.value = -1
    assert lib.idx_topk(ctypes.c_void_p(0x1000), 7, 1, 8, ctypes.c_void_p(0x1000), None, 4, 0,
                        ctypes.c_void_p(0x1000), 8, ctypes.byref(k), None, 0,
                        None) == IDX_EINVAL and k.value == -1  # rejected: untouched
    assert lib.idx_topk_candidates(None, 8, 0, 8, None, None, 2, 4, None, 3, 0, None, 4,
                                   ctypes.byref(k), None) == IDX_OK and k.value == 3


def test_unaligned_pointers_are_rejected(lib):
    """q is read as 16-byte words (idx_score, idx_score_topk), x and the round
    trip of idx_fp4_quant likewise, key rows as 4-byte words: misaligned
    pointers give IDX_EINVAL before any launch."""
    a16, odd8, odd2 = ctypes.c_void_p(0x1000), ctypes.c_void_p(0x1008), ctypes.c_void_p(0x1002)
    # idx_fp4_quant(x, n_rows, rows68, roundtrip, stream)
    assert lib.idx_fp4_quant(odd8, 1, a16, None, None) == IDX_EINVAL
    assert lib.idx_fp4_quant(a16, 1, odd2, None, None) == IDX_EINVAL
    assert lib.idx_fp4_quant(a16, 1, a16, odd8, None) == IDX_EINVAL

    def score(q=a16, kc=a16):
        return lib.idx_score(q, a16, kc, 8, 1, 1, 64, 128, 8, a16, None, 0, 0, a16, 8, None, None)

    def fused(q=a16, kc=a16):
        return lib.idx_score_topk(q, a16, kc, 8, 1, 1, 64, 128, 8, a16, 4, 0, a16, 4, None, 0,
                                  None)

    for call in (score, fused):
        assert call(q=odd8) == IDX_EINVAL
        assert call(kc=odd2) == IDX_EINVAL
    # publish writes 4-byte words of the rows
    assert lib.idx_publish_keys(a16, a16, a16, a16, 10, 1, 1, 512, 128, 64, 1e-6, 7, 4, odd2, 8,
                                8, None) == IDX_EINVAL


@pytest.mark.parametrize("name", ["idx_publish_score", "idx_publish_score_fp8"])
def test_publish_score_checks_both_steps_before_launch(lib, name):
    """idx_publish_score (and its FP8 form) checks the publish's and the
    score's arguments before either step launches, in its one-launch and
    two-launch forms."""
    a16, odd8, odd2 = ctypes.c_void_p(0x1000), ctypes.c_void_p(0x1008), ctypes.c_void_p(0x1002)
    T = 100

    def call(q=a16, kc=a16, sp=4 * (T - 1) + 3, ratio=4, P=400, Din=512, rd=64, eps=1e-6, B=2,
             H=64, D=128, stride=T, ld=T, cl=a16, lat=a16):
        return getattr(lib, name)(lat, a16, a16, a16, P, Din, rd, eps, sp, ratio, q, a16, kc,
                                  stride, B, H, D, T, cl, a16, ld, None, None)

    for sp in (4 * (T - 1) + 3, 4 * 50 + 3, 0):  # one launch, two launches, prefill form
        assert call(sp=sp, q=odd8) == IDX_EINVAL
        assert call(sp=sp, kc=odd2) == IDX_EINVAL
        assert call(sp=sp, ld=T - 1) == IDX_EINVAL
        assert call(sp=sp, stride=T - 1) == IDX_EINVAL
        assert call(sp=sp, cl=None) == IDX_EINVAL
        assert call(sp=sp, lat=None) == IDX_EINVAL
        assert call(sp=sp, H=48) == IDX_EUNSUPPORTED
        assert call(sp=sp, D=64) == IDX_EUNSUPPORTED
        assert call(sp=sp, rd=63) == IDX_EINVAL
        assert call(sp=sp, eps=float("nan")) == IDX_EINVAL
        assert call(sp=sp, B=0) == IDX_OK  # nothing to do
    assert call(ratio=0) == IDX_EINVAL
    assert call(P=4 * (T - 1)) == IDX_EINVAL  # the group's position has no RoPE entry
    assert call(sp=4 * T + 3) == IDX_EINVAL  # its row is past the cache
    assert call(Din=30721) == IDX_EUNSUPPORTED


def test_score_select_blocks_checks_before_launch(lib):
    """idx_score_select_blocks checks the select's arguments (block sizes,
    id row width, workspace size) before the score launches."""
    d = ctypes.c_void_p(0x1000)
    T, R = 65536, 4
    need = lib.idx_select_workspace_size(R, T, 64, 128)

    def call(ctb=64, cbs=128, ld_ids=64, ws=d, ws_bytes=need, ids=d, B=R):
        return lib.idx_score_select_blocks(d, d, d, T, B, 1, 64, 128, T, d, d, T, None, ctb, cbs,
                                           ids, ld_ids, ws, ws_bytes, None)

    assert call(ctb=0) == IDX_EINVAL
    assert call(cbs=0) == IDX_EINVAL
    assert call(ld_ids=63) == IDX_EINVAL  # a row of ids holds min(ctb, nb) = 64
    assert call(ws_bytes=need - 1) == IDX_EINVAL
    assert call(ws=None) == IDX_EINVAL
    assert call(ids=None) == IDX_EINVAL
    assert call(B=0) == IDX_OK  # nothing to do


def test_score_topk_candidates_checks_before_launch(lib):
    """idx_score_topk_candidates checks the top-k's arguments before the
    score launches and leaves k_out untouched when it refuses."""
    d = ctypes.c_void_p(0x1000)
    T, B = 65536, 4

    def call(n_cand=64, cbs=128, ld=8192, ld_out=2048, k=2048, kref=None, Bv=B, Tv=T):
        return lib.idx_score_topk_candidates(d, d, d, Tv, Bv, 1, 64, 128, Tv, d, d, n_cand, cbs,
                                             d, ld, None, k, 0, d, ld_out,
                                             kref if kref is not None else None, None)

    kk = ctypes.c_int32(-1)
    assert call(ld=8191, kref=ctypes.byref(kk)) == IDX_EINVAL and kk.value == -1  # < n_cand * cbs
    assert call(ld_out=2047) == IDX_EINVAL
    assert call(n_cand=0) == IDX_EINVAL
    assert call(k=0) == IDX_EINVAL
    assert call(n_cand=65, ld=65 * 128) == IDX_EUNSUPPORTED  # more than 8192 slots ranked
    assert call(Tv=70000) == IDX_EUNSUPPORTED  # rows past the candidate ranking's width
    assert call(Bv=0, kref=ctypes.byref(kk)) == IDX_OK and kk.value == 2048


def test_paged_entry_points_reject_bad_page_maps(lib):
    """Page pool, page stride and block table are checked before any launch."""
    d = ctypes.c_void_p(0x1000)
    T = 200  # 4 pages of 64 positions

    def score(ps=64 * 68, npg=8, bt=d, bts=4, **kw):
        return lib.idx_score_paged(d, d, d, ps, npg, bt, bts, 1, 1, 64, 128, T, d, None, 0, 0, d,
                                   T, None, None)

    def fused(ps=64 * 68, npg=8, bt=d, bts=4):
        return lib.idx_score_topk_paged(d, d, d, ps, npg, bt, bts, 1, 1, 64, 128, T, d, 64, 0, d,
                                        64, None, 0, None)

    def publish(ps=64 * 68, npg=8, bt=d, bts=4, Tcap=T, sp=4 * 50 - 1):
        return lib.idx_publish_keys_paged(d, d, d, d, 300, 1, 1, 512, 128, 64, 1e-6, sp, 4, d, ps,
                                          npg, bt, bts, Tcap, None)

    for call in (score, fused, publish):
        assert call(bt=None) == IDX_EINVAL  # no block table
        assert call(npg=0) == IDX_EINVAL  # empty page pool
        assert call(ps=64 * 68 - 1) == IDX_EINVAL  # a page shorter than 64 rows
        assert call(bts=3) == IDX_EINVAL  # the table row misses page 3
    assert publish(Tcap=64, sp=4 * 64 + 3) == IDX_EINVAL  # row 64 beyond Tcap
    # nothing to do: no rows
    assert lib.idx_score_paged(d, d, d, 64 * 68, 8, None, 4, 0, 1, 64, 128, T, d, None, 0, 0, d,
                               T, None, None) == IDX_OK
    # level two on pages keeps the row's page ids on chip: T <= 131072
    assert lib.idx_score_paged(d, d, d, 64 * 68, 4096, d, 2049, 1, 1, 64, 128, 131073, d, d, 4,
                               128, d, 131073, None, None) == IDX_EUNSUPPORTED


def test_q_rope_quant_rejects_bad_arguments(lib):
    d = ctypes.c_void_p(0x1000)  # 16-byte aligned, never dereferenced

    def call(q=d, P=64, S=8, D=128, rd=64, sp=0, rt=None):
        return lib.idx_q_rope_quant(q, d, 0.5, d, P, 2, S, 64, D, rd, sp, d, rt, d, None)

    assert call(D=64) == IDX_EUNSUPPORTED
    assert call(rd=63) == IDX_EINVAL
    assert call(rd=130) == IDX_EINVAL
    assert call(sp=57) == IDX_EINVAL  # position 64 not in the table
    assert call(sp=-1) == IDX_EINVAL
    assert call(q=None) == IDX_EINVAL
    assert call(q=ctypes.c_void_p(0x1008)) == IDX_EINVAL  # q not 16-byte aligned
    assert call(rt=ctypes.c_void_p(0x1004)) == IDX_EINVAL  # round trip not 16-byte aligned
    assert call(S=0) == IDX_OK  # nothing to do


def test_score_q4_rejects_unaligned_rows(lib):
    d = ctypes.c_void_p(0x1000)
    odd = ctypes.c_void_p(0x1002)
    assert lib.idx_score_q4(odd, d, d, 8, 1, 1, 64, 128, 8, d, None, 0, 0, d, 8, None,
                            None) == IDX_EINVAL
    assert lib.idx_score_topk_q4(odd, d, d, 8, 1, 1, 64, 128, 8, d, 4, 0, d, 4, None, 0,
                                 None) == IDX_EINVAL
    assert lib.idx_score_q4(None, d, d, 8, 1, 1, 64, 128, 8, d, None, 0, 0, d, 8, None,
                            None) == IDX_EINVAL


def test_tsplit_pairs_and_merge_check_before_launch(lib):
    """idx_topk_pairs and idx_merge_topk refuse their invalid arguments before
    any launch (the pointers below are never dereferenced)."""
    d = ctypes.c_void_p(0x1000)
    kout = ctypes.c_int32(-1)
    ws_need = lib.idx_topk_pairs_workspace_size(4, 32768, 2048)
    assert ws_need >= lib.idx_topk_workspace_size(4, 32768, 2048) + 16

    def pairs(ld=32768, R=4, Tg=32768, start=0, k=2048, ld_out=2048, ws=d, wsb=ws_need,
              pos=d, sc=d):
        return lib.idx_topk_pairs(d, ld, R, Tg, start, d, None, k, pos, sc, ld_out,
                                  ctypes.byref(kout), ws, wsb, None)
    assert pairs(ld=32767) == IDX_EINVAL          # ld < T_slice
    assert pairs(ld_out=2047) == IDX_EINVAL       # ld_out < k_out
    assert pairs(start=-1) == IDX_EINVAL
    assert pairs(start=2 ** 31 - 100) == IDX_EINVAL  # positions past int32
    assert pairs(k=0) == IDX_EINVAL
    assert pairs(ws=None) == IDX_EINVAL
    assert pairs(wsb=ws_need - 1) == IDX_EINVAL
    assert pairs(sc=None) == IDX_EINVAL
    assert pairs(R=0) == IDX_OK and kout.value == 2048  # no rows: k_out only
    assert pairs(Tg=100, ld=100, R=0) == IDX_OK and kout.value == 100

    def merge(G=8, n=2048, stride=4 * 2048, ld=2048, R=4, T=262144, k=2048, ld_out=2048,
              pos=d, sc=d):
        return lib.idx_merge_topk(pos, sc, G, n, stride, ld, R, d, T, k, 0, d, ld_out,
                                  ctypes.byref(kout), None)
    assert merge(G=17) == IDX_EUNSUPPORTED        # 17 x 2048 pairs per row
    assert merge(G=0) == IDX_EINVAL
    assert merge(stride=4 * 2048 - 1) == IDX_EINVAL  # lists of a row would overlap
    assert merge(ld=2047) == IDX_EINVAL           # ld < n
    assert merge(ld_out=2047) == IDX_EINVAL
    assert merge(pos=None) == IDX_EINVAL
    assert merge(k=0) == IDX_EINVAL
    assert merge(R=0) == IDX_OK and kout.value == 2048


def test_publish_score_paged_checks_before_launch(lib):
    """idx_publish_score_paged refuses invalid arguments of either step before
    any launch (the pointers are never dereferenced)."""
    d = ctypes.c_void_p(0x1000)

    def call(H=64, D=128, rd=64, sp=4 * 100 + 3, ps=64 * 68, npg=8, bt=d, bts=2, T=101, ld=101,
             q=d, pages=d, P=512, din=512):
        return lib.idx_publish_score_paged(d, d, d, d, P, din, rd, 1e-6, sp, 4, q, d, pages, ps,
                                           npg, bt, bts, 2, H, D, T, d, d, ld, None, None)
    assert call(H=48) == IDX_EUNSUPPORTED
    assert call(D=64) == IDX_EUNSUPPORTED
    assert call(rd=63) == IDX_EINVAL
    assert call(bt=None) == IDX_EINVAL                 # no block table
    assert call(npg=0) == IDX_EINVAL                   # empty pool
    assert call(ps=64 * 68 - 4) == IDX_EINVAL          # a page shorter than 64 rows
    assert call(ps=64 * 68 + 2) == IDX_EINVAL          # page stride not a multiple of 4
    assert call(bts=1) == IDX_EINVAL                   # the table misses the published row's page
    assert call(ld=100) == IDX_EINVAL                  # scores ld < T
    assert call(q=ctypes.c_void_p(0x1008)) == IDX_EINVAL  # q not 16-byte aligned
    assert call(pages=ctypes.c_void_p(0x1002)) == IDX_EINVAL  # pages not 4-byte aligned
    assert call(P=100) == IDX_EINVAL                   # the key's position not in the RoPE table
    assert call(din=40000) == IDX_EUNSUPPORTED
