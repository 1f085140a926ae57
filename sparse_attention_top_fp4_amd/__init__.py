"""Python binding of the gfx950 DeepSeek-V4.1 Indexer library (libidx.so).

Thin argument marshalling only: every function below checks shapes and
dtypes of torch tensors, passes their device pointers and the current HIP
stream to the C ABI declared in include/idx.h, and raises on a non-zero
status.  All computation happens in the library's HIP kernels.  There is no
fallback: if libidx.so is missing or fails to load, every call raises.

bf16 tensors may be passed as torch.bfloat16 or as torch.uint16/int16 bit
patterns.
"""
from __future__ import annotations

import ctypes
import os

__all__ = ["idx_fp4_quant", "idx_fp8_quant", "idx_score_fp8", "idx_publish_keys_fp8",
           "idx_score", "idx_score_topk", "idx_score_paged",
           "idx_score_topk_paged", "idx_publish_keys_paged", "idx_q_rope_quant",
           "idx_score_q4", "idx_score_topk_q4", "idx_score_qrope", "idx_score_topk_qrope",
           "idx_clear_key_hist", "idx_topk",
           "idx_topk_candidates",
           "idx_topk_workspace_size",
           "idx_select_candidate_blocks", "idx_select_workspace_size", "idx_publish_keys",
           "idx_publish_score", "idx_publish_score_paged", "idx_publish_score_fp8",
           "idx_score_select_blocks",
           "idx_score_topk_candidates",
           "idx_two_level_topk", "idx_topk_pairs", "idx_topk_pairs_workspace_size",
           "idx_merge_topk",
           "idx_yarn_cos_sin", "idx_timing_arm", "idx_timing_read", "library_path",
           "load_library", "IdxError", "ROW_BYTES"]

ROW_BYTES = 68
FP8_ROW_BYTES = 132  # the FP8 cache row: 128 e4m3 bytes + fp32 scale
PAGE_ROWS = 64  # compressed positions per page of a paged key cache
_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libidx.so")
_lib = None


class IdxError(RuntimeError):
    pass


def library_path() -> str:
    return _LIB_PATH


def load_library():
    """Load libidx.so (built by sparse_attention_top_fp4_amd/build.py)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise IdxError(f"HIP library not built: {_LIB_PATH} is missing "
                       "(run python -m sparse_attention_top_fp4_amd.build)")
    L = ctypes.CDLL(_LIB_PATH)
    P, i32, i64, f32, f64, sz = (ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_float,
                                 ctypes.c_double, ctypes.c_size_t)
    L.idx_status_string.argtypes = [i32]
    L.idx_status_string.restype = ctypes.c_char_p
    L.idx_version.restype = ctypes.c_char_p
    L.idx_fp4_quant.argtypes = [P, i64, P, P, P]
    L.idx_score.argtypes = [P, P, P, i64, i32, i32, i32, i32, i32, P, P, i32, i32, P, i64, P, P]
    L.idx_score_topk.argtypes = [P, P, P, i64, i32, i32, i32, i32, i32, P, i32, ctypes.c_int32,
                                 P, i64, P, i64, P]
    L.idx_clear_key_hist.argtypes = [P, i32, P]
    L.idx_topk_workspace_size.argtypes = [i32, i32, i32]
    L.idx_topk_workspace_size.restype = sz
    L.idx_topk.argtypes = [P, i64, i32, i32, P, P, i32, ctypes.c_int32, P, i64, P, P, sz, P]
    L.idx_topk_candidates.argtypes = [P, i64, i32, i32, P, P, i32, i32, P, i32, ctypes.c_int32,
                                      P, i64, P, P]
    L.idx_select_workspace_size.argtypes = [i32, i32, i32, i32]
    L.idx_select_workspace_size.restype = sz
    L.idx_select_candidate_blocks.argtypes = [P, i64, i32, i32, P, i32, i32, P, i64, P, sz, P]
    L.idx_publish_keys.argtypes = [P, P, P, P, i32, i32, i32, i32, i32, i32, f32, i32, i32, P, i64,
                                   i32, P]
    L.idx_score_paged.argtypes = [P, P, P, i64, i32, P, i64, i32, i32, i32, i32, i32, P, P, i32,
                                  i32, P, i64, P, P]
    L.idx_score_topk_paged.argtypes = [P, P, P, i64, i32, P, i64, i32, i32, i32, i32, i32, P, i32,
                                       ctypes.c_int32, P, i64, P, i64, P]
    L.idx_publish_keys_paged.argtypes = [P, P, P, P, i32, i32, i32, i32, i32, i32, f32, i32, i32,
                                         P, i64, i32, P, i64, i32, P]
    L.idx_q_rope_quant.argtypes = [P, P, f32, P, i32, i32, i32, i32, i32, i32, i32, P, P, P, P]
    L.idx_score_qrope.argtypes = [P, P, f32, P, i32, i32, i32, P, i64, i32, i32, i32, i32, i32, P,
                                  P, i64, P, P]
    L.idx_score_topk_qrope.argtypes = [P, P, f32, P, i32, i32, i32, P, i64, i32, i32, i32, i32,
                                       i32, P, i32, ctypes.c_int32, P, i64, P, i64, P]
    L.idx_score_q4.argtypes = L.idx_score.argtypes
    L.idx_score_topk_q4.argtypes = L.idx_score_topk.argtypes
    L.idx_yarn_cos_sin.argtypes = [i32, i32, f64, f64, i32, f64, f64, P]
    L.idx_fp8_quant.argtypes = [P, i64, P, P, P]
    L.idx_score_fp8.argtypes = L.idx_score.argtypes
    L.idx_publish_keys_fp8.argtypes = L.idx_publish_keys.argtypes
    L.idx_score_topk_candidates.argtypes = [P, P, P, i64, i32, i32, i32, i32, i32, P, P, i32, i32,
                                            P, i64, P, i32, ctypes.c_int32, P, i64, P, P]
    L.idx_two_level_topk.argtypes = [P, i64, P, P, i64, P, sz, P, P, P, i64, i32, i32, i32, i32, i32,
                                     P, P, i32, i32, P, i64, P, i32, ctypes.c_int32, P, i64, P]
    L.idx_score_select_blocks.argtypes = [P, P, P, i64, i32, i32, i32, i32, i32, P, P, i64, P,
                                          i32, i32, P, i64, P, sz, P]
    L.idx_publish_score.argtypes = [P, P, P, P, i32, i32, i32, f32, i32, i32, P, P, P, i64, i32,
                                    i32, i32, i32, P, P, i64, P, P]
    L.idx_publish_score_fp8.argtypes = L.idx_publish_score.argtypes
    L.idx_publish_score_paged.argtypes = [P, P, P, P, i32, i32, i32, f32, i32, i32, P, P, P, i64,
                                          i32, P, i64, i32, i32, i32, i32, P, P, i64, P, P]
    L.idx_topk_pairs_workspace_size.argtypes = [i32, i32, i32]
    L.idx_topk_pairs_workspace_size.restype = sz
    L.idx_topk_pairs.argtypes = [P, i64, i32, i32, i32, P, P, i32, P, P, i64, P, P, sz, P]
    L.idx_merge_topk.argtypes = [P, P, i32, i32, i64, i64, i32, P, i32, i32, ctypes.c_int32, P,
                                 i64, P, P]
    L.idx_probe_stream_read.argtypes = [P, i64, i32, P, ctypes.POINTER(f32), P]
    L.idx_probe_mfma_fp4.argtypes = [i32, i32, P, ctypes.POINTER(f64), ctypes.POINTER(f32), P]
    L.idx_probe_bf16_convert.argtypes = [P, ctypes.POINTER(ctypes.c_ulonglong), P]
    L.idx_probe_bf16_convert.restype = i32
    L.idx_timing_arm.argtypes = [i32]
    L.idx_timing_read.argtypes = [i32, ctypes.POINTER(f32)]
    for name in ("idx_fp4_quant", "idx_score", "idx_score_topk", "idx_clear_key_hist", "idx_topk",
                 "idx_topk_candidates",
                 "idx_select_candidate_blocks",
                 "idx_publish_keys", "idx_yarn_cos_sin", "idx_timing_arm", "idx_timing_read",
                 "idx_score_paged", "idx_score_topk_paged", "idx_publish_keys_paged",
                 "idx_q_rope_quant", "idx_score_q4", "idx_score_topk_q4",
                 "idx_probe_stream_read", "idx_probe_mfma_fp4", "idx_fp8_quant",
                 "idx_score_fp8", "idx_publish_keys_fp8", "idx_publish_score",
                 "idx_score_select_blocks", "idx_score_topk_candidates", "idx_two_level_topk",
                 "idx_score_qrope", "idx_score_topk_qrope", "idx_topk_pairs", "idx_merge_topk",
                 "idx_publish_score_paged", "idx_publish_score_fp8"):
        getattr(L, name).restype = i32
    _lib = L
    return L


def _check(status: int, what: str):
    if status != 0:
        msg = load_library().idx_status_string(status).decode()
        raise IdxError(f"{what}: {msg}")


class BoundCall:
    """One library call with every argument but the stream marshalled once:
    calling it issues the call again on the given stream (a raw hipStream_t
    handle, or None for torch's current stream) and raises on a non-zero
    status.  For loops that repeat the same calls on the same buffers, where
    re-checking and re-converting the tensors would cost more host time than
    the kernels take."""

    __slots__ = ("_fn", "_args", "_what", "_keep")

    def __init__(self, fn, args, what, keep=()):
        # keep: tensors the call's pointers refer to that the caller does not
        # hold itself (a workspace allocated by the wrapper)
        self._fn, self._args, self._what, self._keep = fn, args, what, keep

    def __call__(self, stream=None):
        if stream is None:
            stream = _stream(None)
        st = self._fn(*self._args, stream)
        if st:
            _check(st, self._what)


def _issue(name, args, stream, what, bind, keep=()):
    """Call library function `name` with `args` and the stream, or (bind)
    return the call as a BoundCall without issuing it.  A bound call holds
    raw device pointers: the caller keeps the tensors alive while it uses
    the call."""
    fn = getattr(load_library(), name)
    if bind:
        return BoundCall(fn, tuple(args), what, keep)
    _check(fn(*args, _stream(stream)), what)
    return None


def current_stream_handle():
    """The raw handle of torch's current stream, for BoundCall."""
    return _stream(None)


def _torch():
    import torch
    return torch


def _stream(stream):
    torch = _torch()
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dev(t, name, dtypes, ndim=None):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if dtypes is not None and t.dtype not in dtypes:
        raise TypeError(f"{name}: dtype {t.dtype} not in {dtypes}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name}: expected {ndim} dims, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _bf16_types():
    torch = _torch()
    return (torch.bfloat16, torch.uint16, torch.int16)


def idx_fp4_quant(x, rows68, roundtrip=None, stream=None, bind=False):
    """x [n, 128] bf16 -> rows68 [n, 68] uint8 (+ roundtrip [n, 128] bf16)."""
    torch = _torch()
    _dev(x, "x", _bf16_types())
    _dev(rows68, "rows68", (torch.uint8,))
    n = x.numel() // 128
    if x.shape[-1] != 128 or rows68.numel() != n * ROW_BYTES:
        raise ValueError("x must be [..., 128] and rows68 [..., 68] with the same rows")
    if roundtrip is not None:
        _dev(roundtrip, "roundtrip", _bf16_types())
        if roundtrip.numel() != x.numel():
            raise ValueError("roundtrip must match x")
    return _issue("idx_fp4_quant", (_ptr(x), n, _ptr(rows68), _ptr(roundtrip)), stream,
                  "idx_fp4_quant", bind)


def idx_score(q, w, k_cache, B, S, T, compress_lens, scores, cand_blocks=None,
              cand_block_size=0, key_hist=None, stream=None, bind=False):
    """q [B*S, H, 128] bf16, w [B*S, H] bf16, k_cache [B, Tcap, 68] uint8,
    compress_lens [B*S] int32, scores [B*S, ld] float32 (ld >= T),
    cand_blocks [B*S, n_cand] int32 or None, key_hist [B*S, 2048] int32
    (uint32 counts, added to; clear with idx_clear_key_hist) or None."""
    torch = _torch()
    _dev(q, "q", _bf16_types(), 3)
    _dev(w, "w", _bf16_types(), 2)
    _dev(k_cache, "k_cache", (torch.uint8,), 3)
    _dev(compress_lens, "compress_lens", (torch.int32,), 1)
    _dev(scores, "scores", (torch.float32,), 2)
    R, H, D = q.shape
    if R != B * S or tuple(w.shape) != (R, H) or compress_lens.shape[0] != R:
        raise ValueError("q/w/compress_lens rows must be B*S")
    if k_cache.shape[0] < B or k_cache.shape[2] != ROW_BYTES or scores.shape[0] != R:
        raise ValueError("k_cache must be [>=B, Tcap, 68] and scores [B*S, ld]")
    n_cand = 0
    if cand_blocks is not None:
        _dev(cand_blocks, "cand_blocks", (torch.int32,), 2)
        if cand_blocks.shape[0] != R:
            raise ValueError("cand_blocks must have B*S rows")
        n_cand = cand_blocks.shape[1]
    if key_hist is not None:
        _dev(key_hist, "key_hist", (torch.int32,), 2)
        if tuple(key_hist.shape) != (R, 2048):
            raise ValueError("key_hist must be [B*S, 2048]")
    return _issue("idx_score", (_ptr(q), _ptr(w), _ptr(k_cache), k_cache.shape[1], B, S, H, D,
                                    T, _ptr(compress_lens), _ptr(cand_blocks), n_cand,
                                    cand_block_size, _ptr(scores), scores.shape[1],
                                    _ptr(key_hist)), stream, "idx_score", bind)


def idx_fp8_quant(x, rows132, roundtrip=None, stream=None, bind=False):
    """x [n, 128] bf16 -> rows132 [n, 132] uint8 FP8 rows (+ roundtrip)."""
    torch = _torch()
    _dev(x, "x", _bf16_types())
    _dev(rows132, "rows132", (torch.uint8,))
    n = x.numel() // 128
    if x.shape[-1] != 128 or rows132.numel() != n * FP8_ROW_BYTES:
        raise ValueError("x must be [..., 128] and rows132 [..., 132] with the same rows")
    if roundtrip is not None:
        _dev(roundtrip, "roundtrip", _bf16_types())
        if roundtrip.numel() != x.numel():
            raise ValueError("roundtrip must match x")
    return _issue("idx_fp8_quant", (_ptr(x), n, _ptr(rows132), _ptr(roundtrip)), stream,
                  "idx_fp8_quant", bind)


def idx_score_fp8(q, w, k_cache, B, S, T, compress_lens, scores, cand_blocks=None,
                  cand_block_size=0, key_hist=None, stream=None, bind=False):
    """idx_score on the FP8 cache: k_cache [B, Tcap, 132] uint8."""
    torch = _torch()
    _dev(q, "q", _bf16_types(), 3)
    _dev(w, "w", _bf16_types(), 2)
    _dev(k_cache, "k_cache", (torch.uint8,), 3)
    _dev(compress_lens, "compress_lens", (torch.int32,), 1)
    _dev(scores, "scores", (torch.float32,), 2)
    R, H, D = q.shape
    if R != B * S or tuple(w.shape) != (R, H) or compress_lens.shape[0] != R:
        raise ValueError("q/w/compress_lens rows must be B*S")
    if k_cache.shape[0] < B or k_cache.shape[2] != FP8_ROW_BYTES or scores.shape[0] != R:
        raise ValueError("k_cache must be [>=B, Tcap, 132] and scores [B*S, ld]")
    n_cand = 0
    if cand_blocks is not None:
        _dev(cand_blocks, "cand_blocks", (torch.int32,), 2)
        if cand_blocks.shape[0] != R:
            raise ValueError("cand_blocks must have B*S rows")
        n_cand = cand_blocks.shape[1]
    if key_hist is not None:
        _dev(key_hist, "key_hist", (torch.int32,), 2)
        if tuple(key_hist.shape) != (R, 2048):
            raise ValueError("key_hist must be [B*S, 2048]")
    return _issue("idx_score_fp8", (_ptr(q), _ptr(w), _ptr(k_cache), k_cache.shape[1], B, S, H,
                                    D, T, _ptr(compress_lens), _ptr(cand_blocks), n_cand,
                                    cand_block_size, _ptr(scores), scores.shape[1],
                                    _ptr(key_hist)), stream, "idx_score_fp8", bind)


def idx_publish_keys_fp8(latent, wk, gamma, cos_sin, start_pos, ratio, eps, k_cache, rd=64,
                         stream=None, bind=False):
    """idx_publish_keys into an FP8 cache k_cache [B', Tcap, 132] uint8."""
    torch = _torch()
    _dev(latent, "latent", _bf16_types(), 3)
    _dev(wk, "wk", _bf16_types(), 2)
    _dev(gamma, "gamma", (torch.float32,), 1)
    _dev(cos_sin, "cos_sin", (torch.float32,), 3)
    _dev(k_cache, "k_cache", (torch.uint8,), 3)
    B, G, Din = latent.shape
    D = wk.shape[0]
    if (wk.shape[1] != Din or gamma.shape[0] != D or k_cache.shape[0] < B
            or k_cache.shape[2] != FP8_ROW_BYTES):
        raise ValueError("shape mismatch in idx_publish_keys_fp8")
    return _issue("idx_publish_keys_fp8", (_ptr(latent), _ptr(wk), _ptr(gamma), _ptr(cos_sin),
                                           cos_sin.shape[0], B, G, Din, D, rd, eps, start_pos,
                                           ratio, _ptr(k_cache), k_cache.shape[1],
                                           k_cache.shape[1]), stream, "idx_publish_keys_fp8",
                  bind)


def idx_score_q4(q_rows, w, k_cache, B, S, T, compress_lens, scores, cand_blocks=None,
                 cand_block_size=0, key_hist=None, stream=None, bind=False):
    """idx_score with the query heads already quantised: q_rows [B*S, H, 68]
    uint8 (from idx_q_rope_quant or idx_fp4_quant)."""
    torch = _torch()
    _dev(q_rows, "q_rows", (torch.uint8,), 3)
    _dev(w, "w", _bf16_types(), 2)
    _dev(k_cache, "k_cache", (torch.uint8,), 3)
    _dev(compress_lens, "compress_lens", (torch.int32,), 1)
    _dev(scores, "scores", (torch.float32,), 2)
    R, H, rb = q_rows.shape
    if rb != ROW_BYTES or R != B * S or tuple(w.shape) != (R, H) or compress_lens.shape[0] != R:
        raise ValueError("q_rows must be [B*S, H, 68] and w/compress_lens rows B*S")
    if k_cache.shape[0] < B or k_cache.shape[2] != ROW_BYTES or scores.shape[0] != R:
        raise ValueError("k_cache must be [>=B, Tcap, 68] and scores [B*S, ld]")
    n_cand = 0
    if cand_blocks is not None:
        _dev(cand_blocks, "cand_blocks", (torch.int32,), 2)
        if cand_blocks.shape[0] != R:
            raise ValueError("cand_blocks must have B*S rows")
        n_cand = cand_blocks.shape[1]
    if key_hist is not None:
        _dev(key_hist, "key_hist", (torch.int32,), 2)
        if tuple(key_hist.shape) != (R, 2048):
            raise ValueError("key_hist must be [B*S, 2048]")
    return _issue("idx_score_q4", (_ptr(q_rows), _ptr(w), _ptr(k_cache), k_cache.shape[1], B,
                                       S, H, 128, T, _ptr(compress_lens), _ptr(cand_blocks),
                                       n_cand, cand_block_size, _ptr(scores), scores.shape[1],
                                       _ptr(key_hist)), stream, "idx_score_q4", bind)


def idx_score_topk_q4(q_rows, w, k_cache, B, S, T, compress_lens, index_topk, offset, out,
                      scores=None, stream=None, bind=False):
    """idx_score_topk with the query heads already quantised: q_rows
    [B*S, H, 68] uint8."""
    torch = _torch()
    _dev(q_rows, "q_rows", (torch.uint8,), 3)
    _dev(w, "w", _bf16_types(), 2)
    _dev(k_cache, "k_cache", (torch.uint8,), 3)
    _dev(compress_lens, "compress_lens", (torch.int32,), 1)
    _dev(out, "out", (torch.int32,), 2)
    R, H, rb = q_rows.shape
    if rb != ROW_BYTES or R != B * S or tuple(w.shape) != (R, H) or compress_lens.shape[0] != R:
        raise ValueError("q_rows must be [B*S, H, 68] and w/compress_lens rows B*S")
    if k_cache.shape[0] < B or k_cache.shape[2] != ROW_BYTES or out.shape[0] != R:
        raise ValueError("k_cache must be [>=B, Tcap, 68] and out [B*S, ld_out]")
    ld = 0
    if scores is not None:
        _dev(scores, "scores", (torch.float32,), 2)
        if scores.shape[0] != R:
            raise ValueError("scores must be [B*S, ld]")
        ld = scores.shape[1]
    return _issue("idx_score_topk_q4", (_ptr(q_rows), _ptr(w), _ptr(k_cache),
                                            k_cache.shape[1], B, S, H, 128, T,
                                            _ptr(compress_lens), index_topk, offset, _ptr(out),
                                            out.shape[1], _ptr(scores), ld), stream,
                  "idx_score_topk_q4", bind)


def idx_score_topk(q, w, k_cache, B, S, T, compress_lens, index_topk, offset, out, scores=None,
                   stream=None, bind=False):
    """idx_score then idx_topk in one launch, for T <= 8192: q [B*S, H, 128]
    bf16, w [B*S, H] bf16, k_cache [B, Tcap, 68] uint8, compress_lens [B*S]
    int32, out [B*S, ld_out] int32 (ld_out >= min(index_topk, T)); scores
    [B*S, ld] float32 also receives the scores when given."""
    torch = _torch()
    _dev(q, "q", _bf16_types(), 3)
    _dev(w, "w", _bf16_types(), 2)
    _dev(k_cache, "k_cache", (torch.uint8,), 3)
    _dev(compress_lens, "compress_lens", (torch.int32,), 1)
    _dev(out, "out", (torch.int32,), 2)
    R, H, D = q.shape
    if R != B * S or tuple(w.shape) != (R, H) or compress_lens.shape[0] != R:
        raise ValueError("q/w/compress_lens rows must be B*S")
    if k_cache.shape[0] < B or k_cache.shape[2] != ROW_BYTES or out.shape[0] != R:
        raise ValueError("k_cache must be [>=B, Tcap, 68] and out [B*S, ld_out]")
    ld = 0
    if scores is not None:
        _dev(scores, "scores", (torch.float32,), 2)
        if scores.shape[0] != R:
            raise ValueError("scores must be [B*S, ld]")
        ld = scores.shape[1]
    return _issue("idx_score_topk", (_ptr(q), _ptr(w), _ptr(k_cache), k_cache.shape[1], B, S,
                                         H, D, T, _ptr(compress_lens), index_topk, offset,
                                         _ptr(out), out.shape[1], _ptr(scores), ld), stream,
                  "idx_score_topk", bind)


def _pages(k_pages, block_table, B):
    """k_pages [n_pages, page_bytes] or [n_pages, 64, 68] uint8 (page_bytes >=
    64 * 68), block_table [>= B, bt_stride] int32 -> (page_stride, n_pages,
    bt_stride)."""
    torch = _torch()
    _dev(k_pages, "k_pages", (torch.uint8,))
    _dev(block_table, "block_table", (torch.int32,), 2)
    if k_pages.dim() not in (2, 3) or block_table.shape[0] < B:
        raise ValueError("k_pages must be [n_pages, page_bytes] or [n_pages, 64, 68] and "
                         "block_table [>=B, bt_stride]")
    return k_pages.stride(0), k_pages.shape[0], block_table.shape[1]


def idx_score_paged(q, w, k_pages, block_table, B, S, T, compress_lens, scores, cand_blocks=None,
                    cand_block_size=0, key_hist=None, stream=None, bind=False):
    """idx_score on a paged key cache: row t of sequence b in slot t % 64 of
    page block_table[b, t // 64] of k_pages."""
    torch = _torch()
    _dev(q, "q", _bf16_types(), 3)
    _dev(w, "w", _bf16_types(), 2)
    _dev(compress_lens, "compress_lens", (torch.int32,), 1)
    _dev(scores, "scores", (torch.float32,), 2)
    R, H, D = q.shape
    if R != B * S or tuple(w.shape) != (R, H) or compress_lens.shape[0] != R:
        raise ValueError("q/w/compress_lens rows must be B*S")
    if scores.shape[0] != R:
        raise ValueError("scores must be [B*S, ld]")
    if key_hist is not None:
        _dev(key_hist, "key_hist", (torch.int32,), 2)
        if tuple(key_hist.shape) != (R, 2048):
            raise ValueError("key_hist must be [B*S, 2048]")
    n_cand = 0
    if cand_blocks is not None:
        _dev(cand_blocks, "cand_blocks", (torch.int32,), 2)
        if cand_blocks.shape[0] != R:
            raise ValueError("cand_blocks must have B*S rows")
        n_cand = cand_blocks.shape[1]
    ps, npg, bts = _pages(k_pages, block_table, B)
    return _issue("idx_score_paged", (_ptr(q), _ptr(w), _ptr(k_pages), ps, npg,
                                          _ptr(block_table), bts, B, S, H, D, T,
                                          _ptr(compress_lens), _ptr(cand_blocks), n_cand,
                                          cand_block_size, _ptr(scores), scores.shape[1],
                                          _ptr(key_hist)), stream, "idx_score_paged", bind)


def idx_score_topk_paged(q, w, k_pages, block_table, B, S, T, compress_lens, index_topk, offset,
                         out, scores=None, stream=None, bind=False):
    """idx_score_topk on a paged key cache (pages as for idx_score_paged)."""
    torch = _torch()
    _dev(q, "q", _bf16_types(), 3)
    _dev(w, "w", _bf16_types(), 2)
    _dev(compress_lens, "compress_lens", (torch.int32,), 1)
    _dev(out, "out", (torch.int32,), 2)
    R, H, D = q.shape
    if R != B * S or tuple(w.shape) != (R, H) or compress_lens.shape[0] != R:
        raise ValueError("q/w/compress_lens rows must be B*S")
    if out.shape[0] != R:
        raise ValueError("out must be [B*S, ld_out]")
    ld = 0
    if scores is not None:
        _dev(scores, "scores", (torch.float32,), 2)
        if scores.shape[0] != R:
            raise ValueError("scores must be [B*S, ld]")
        ld = scores.shape[1]
    ps, npg, bts = _pages(k_pages, block_table, B)
    return _issue("idx_score_topk_paged", (_ptr(q), _ptr(w), _ptr(k_pages), ps, npg,
                                               _ptr(block_table), bts, B, S, H, D, T,
                                               _ptr(compress_lens), index_topk, offset,
                                               _ptr(out), out.shape[1], _ptr(scores), ld), stream,
                  "idx_score_topk_paged", bind)


def idx_publish_keys_paged(latent, wk, gamma, cos_sin, start_pos, ratio, eps, k_pages,
                           block_table, Tcap, rd=64, stream=None, bind=False):
    """idx_publish_keys into a paged key cache of Tcap rows per sequence."""
    torch = _torch()
    _dev(latent, "latent", _bf16_types(), 3)
    _dev(wk, "wk", _bf16_types(), 2)
    _dev(gamma, "gamma", (torch.float32,), 1)
    _dev(cos_sin, "cos_sin", (torch.float32,), 3)
    B, G, Din = latent.shape
    D = wk.shape[0]
    if wk.shape[1] != Din or gamma.shape[0] != D:
        raise ValueError("shape mismatch in idx_publish_keys_paged")
    ps, npg, bts = _pages(k_pages, block_table, B)
    return _issue("idx_publish_keys_paged", (_ptr(latent), _ptr(wk), _ptr(gamma),
                                                 _ptr(cos_sin), cos_sin.shape[0], B, G, Din, D,
                                                 rd, eps, start_pos, ratio, _ptr(k_pages), ps,
                                                 npg, _ptr(block_table), bts, Tcap), stream,
                  "idx_publish_keys_paged", bind)


def idx_q_rope_quant(q, w_raw, w_scale, cos_sin, start_pos, S, q_rows, w_out,
                     q_roundtrip=None, rd=64, stream=None, bind=False):
    """Query RoPE + fp4 quantise + weight scaling: q [B*S, H, 128] bf16
    (before RoPE), w_raw [B*S, H] bf16, cos_sin [P, rd/2, 2] float32, rows
    r = b*S + s at position start_pos + s; q_rows [B*S, H, 68] uint8,
    w_out [B*S, H] bf16, q_roundtrip [B*S, H, 128] bf16 or None."""
    torch = _torch()
    _dev(q, "q", _bf16_types(), 3)
    _dev(w_raw, "w_raw", _bf16_types(), 2)
    _dev(cos_sin, "cos_sin", (torch.float32,), 3)
    _dev(q_rows, "q_rows", (torch.uint8,), 3)
    _dev(w_out, "w_out", _bf16_types(), 2)
    R, H, D = q.shape
    if R % S or tuple(w_raw.shape) != (R, H) or tuple(w_out.shape) != (R, H):
        raise ValueError("q/w rows must be B*S")
    if tuple(q_rows.shape) != (R, H, ROW_BYTES):
        raise ValueError("q_rows must be [B*S, H, 68]")
    if q_roundtrip is not None:
        _dev(q_roundtrip, "q_roundtrip", _bf16_types(), 3)
        if tuple(q_roundtrip.shape) != (R, H, D):
            raise ValueError("q_roundtrip must be shaped like q")
    return _issue("idx_q_rope_quant", (_ptr(q), _ptr(w_raw), w_scale, _ptr(cos_sin),
                                           cos_sin.shape[0], R // S, S, H, D, rd, start_pos,
                                           _ptr(q_rows), _ptr(q_roundtrip), _ptr(w_out)), stream,
                  "idx_q_rope_quant", bind)


def _qstep_args(q, w_raw, cos_sin, B, S):
    torch = _torch()
    _dev(q, "q", _bf16_types(), 3)
    _dev(w_raw, "w_raw", _bf16_types(), 2)
    _dev(cos_sin, "cos_sin", (torch.float32,), 3)
    R, H, D = q.shape
    if R != B * S or tuple(w_raw.shape) != (R, H):
        raise ValueError("q/w_raw rows must be B*S")
    return R, H, D


def idx_score_qrope(q, w_raw, w_scale, cos_sin, start_pos, k_cache, B, S, T, compress_lens,
                    scores, key_hist=None, rd=64, stream=None, bind=False):
    """The query step (idx_q_rope_quant) inside the score launch: q [B*S, H,
    128] bf16 before RoPE, w_raw [B*S, H] bf16, w_scale, cos_sin [P, rd/2, 2]
    float32; rows r = b*S + s at position start_pos + s.  Other arguments
    as idx_score (no candidate blocks)."""
    torch = _torch()
    R, H, D = _qstep_args(q, w_raw, cos_sin, B, S)
    _dev(k_cache, "k_cache", (torch.uint8,), 3)
    _dev(compress_lens, "compress_lens", (torch.int32,), 1)
    _dev(scores, "scores", (torch.float32,), 2)
    if compress_lens.shape[0] != R or scores.shape[0] != R:
        raise ValueError("compress_lens and scores must have B*S rows")
    if k_cache.shape[0] < B or k_cache.shape[2] != ROW_BYTES:
        raise ValueError("k_cache must be [>=B, Tcap, 68]")
    if key_hist is not None:
        _dev(key_hist, "key_hist", (torch.int32,), 2)
        if tuple(key_hist.shape) != (R, 2048):
            raise ValueError("key_hist must be [B*S, 2048]")
    return _issue("idx_score_qrope", (_ptr(q), _ptr(w_raw), w_scale, _ptr(cos_sin),
                                          cos_sin.shape[0], rd, start_pos, _ptr(k_cache),
                                          k_cache.shape[1], B, S, H, D, T, _ptr(compress_lens),
                                          _ptr(scores), scores.shape[1], _ptr(key_hist)), stream,
                  "idx_score_qrope", bind)


def idx_score_topk_qrope(q, w_raw, w_scale, cos_sin, start_pos, k_cache, B, S, T, compress_lens,
                         index_topk, offset, out, scores=None, rd=64, stream=None, bind=False):
    """idx_score_topk with the query step in its launch (arguments as
    idx_score_qrope and idx_score_topk)."""
    torch = _torch()
    R, H, D = _qstep_args(q, w_raw, cos_sin, B, S)
    _dev(k_cache, "k_cache", (torch.uint8,), 3)
    _dev(compress_lens, "compress_lens", (torch.int32,), 1)
    _dev(out, "out", (torch.int32,), 2)
    if compress_lens.shape[0] != R or out.shape[0] != R:
        raise ValueError("compress_lens and out must have B*S rows")
    if k_cache.shape[0] < B or k_cache.shape[2] != ROW_BYTES:
        raise ValueError("k_cache must be [>=B, Tcap, 68]")
    ld = 0
    if scores is not None:
        _dev(scores, "scores", (torch.float32,), 2)
        if scores.shape[0] != R:
            raise ValueError("scores must be [B*S, ld]")
        ld = scores.shape[1]
    return _issue("idx_score_topk_qrope", (_ptr(q), _ptr(w_raw), w_scale, _ptr(cos_sin),
                                               cos_sin.shape[0], rd, start_pos, _ptr(k_cache),
                                               k_cache.shape[1], B, S, H, D, T,
                                               _ptr(compress_lens), index_topk, offset, _ptr(out),
                                               out.shape[1], _ptr(scores), ld), stream,
                  "idx_score_topk_qrope", bind)


def idx_clear_key_hist(key_hist, stream=None, bind=False):
    """Zero a [R, 2048] int32 score histogram before idx_score adds to it."""
    torch = _torch()
    _dev(key_hist, "key_hist", (torch.int32,), 2)
    if key_hist.shape[1] != 2048:
        raise ValueError("key_hist must be [R, 2048]")
    return _issue("idx_clear_key_hist", (_ptr(key_hist), key_hist.shape[0]), stream,
                  "idx_clear_key_hist", bind)


def idx_topk_workspace_size(R, T, index_topk) -> int:
    return int(load_library().idx_topk_workspace_size(R, T, index_topk))


def idx_topk(scores, T, compress_lens, index_topk, offset, out, workspace=None, key_hist=None,
             stream=None, bind=False):
    """scores [R, ld] float32, compress_lens [R] int32, out [R, ld_out] int32
    (ld_out >= min(index_topk, T)).  workspace: uint8 device tensor of at
    least idx_topk_workspace_size bytes, allocated here when None.
    key_hist: the [R, 2048] histogram idx_score produced for these scores;
    the call resets it to zero.  Returns k_out = min(index_topk, T), the
    width written per row."""
    torch = _torch()
    _dev(scores, "scores", (torch.float32,), 2)
    _dev(compress_lens, "compress_lens", (torch.int32,), 1)
    _dev(out, "out", (torch.int32,), 2)
    R = scores.shape[0]
    need = idx_topk_workspace_size(R, T, index_topk)
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=scores.device)
    wsb = 0 if workspace is None else workspace.numel() * workspace.element_size()
    if key_hist is not None:
        _dev(key_hist, "key_hist", (torch.int32,), 2)
        if tuple(key_hist.shape) != (R, 2048):
            raise ValueError("key_hist must be [R, 2048]")
    kout = ctypes.c_int32(-1)
    bound = _issue("idx_topk", (_ptr(scores), scores.shape[1], R, T, _ptr(compress_lens),
                                _ptr(key_hist), index_topk, offset, _ptr(out), out.shape[1],
                                ctypes.byref(kout), _ptr(workspace), wsb), stream, "idx_topk",
                   bind, keep=(workspace,))
    return bound if bind else kout.value


def idx_topk_pairs_workspace_size(R: int, T_slice: int, index_topk: int) -> int:
    return int(load_library().idx_topk_pairs_workspace_size(R, T_slice, index_topk))


def idx_topk_pairs(scores, slice_start, T_slice, compress_lens, index_topk, pos_out, score_out,
                   workspace=None, key_hist=None, stream=None, bind=False):
    """The top-k of the slice [slice_start, slice_start + T_slice) of each row
    of scores [R, ld] float32, as (position, score) pairs: pos_out [R, ld_out]
    int32 gets the slice's top min(index_topk, T_slice) row positions in
    ascending order (-1 where not below compress_lens [R], the rows' own
    lengths), score_out [R, ld_out] float32 their scores (-inf for -1).
    key_hist: a histogram idx_score made of this slice with the slice's
    compress_lens, or None.  Returns the width written per row."""
    torch = _torch()
    _dev(scores, "scores", (torch.float32,), 2)
    _dev(compress_lens, "compress_lens", (torch.int32,), 1)
    _dev(pos_out, "pos_out", (torch.int32,), 2)
    _dev(score_out, "score_out", (torch.float32,), 2)
    R, ld = scores.shape
    if not 0 <= slice_start <= ld or T_slice < 0 or slice_start + T_slice > ld:
        raise ValueError("the slice must lie inside the rows of scores")
    if compress_lens.shape[0] != R or pos_out.shape[0] != R or score_out.shape != pos_out.shape:
        raise ValueError("scores, compress_lens, pos_out and score_out need the same rows")
    need = idx_topk_pairs_workspace_size(R, T_slice, index_topk)
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=scores.device)
    wsb = 0 if workspace is None else workspace.numel() * workspace.element_size()
    if key_hist is not None:
        _dev(key_hist, "key_hist", (torch.int32,), 2)
        if tuple(key_hist.shape) != (R, 2048):
            raise ValueError("key_hist must be [R, 2048]")
    kout = ctypes.c_int32(-1)
    first = ctypes.c_void_p(scores.data_ptr() + 4 * slice_start)
    bound = _issue("idx_topk_pairs", (first, ld, R, T_slice, slice_start, _ptr(compress_lens),
                                      _ptr(key_hist), index_topk, _ptr(pos_out), _ptr(score_out),
                                      pos_out.shape[1], ctypes.byref(kout), _ptr(workspace), wsb),
                   stream, "idx_topk_pairs", bind, keep=(workspace,))
    return bound if bind else kout.value


def idx_merge_topk(pos, score, compress_lens, T, index_topk, offset, out, stream=None,
                   bind=False):
    """The row top-k from the slices' pairs: pos [G, R, n] int32 and score
    [G, R, n] float32 hold list g of row r (idx_topk_pairs of slice g, the
    slices in position order; shorter lists padded with -1); out [R, ld_out]
    int32 gets what idx_topk gives on the rows of width T with compress_lens
    [R].  Returns k_out = min(index_topk, T)."""
    torch = _torch()
    _dev(pos, "pos", (torch.int32,), 3)
    _dev(score, "score", (torch.float32,), 3)
    _dev(compress_lens, "compress_lens", (torch.int32,), 1)
    _dev(out, "out", (torch.int32,), 2)
    G, R, n = pos.shape
    if tuple(score.shape) != (G, R, n):
        raise ValueError("pos and score must have the same shape")
    if compress_lens.shape[0] != R or out.shape[0] != R:
        raise ValueError("pos, compress_lens and out need the same rows")
    kout = ctypes.c_int32(-1)
    bound = _issue("idx_merge_topk", (_ptr(pos), _ptr(score), G, n, R * n, n, R,
                                      _ptr(compress_lens), T, index_topk, offset, _ptr(out),
                                      out.shape[1], ctypes.byref(kout)),
                   stream, "idx_merge_topk", bind)
    return bound if bind else kout.value


def idx_topk_candidates(scores, T, compress_lens, cand_blocks, cand_block_size, index_topk,
                        offset, out, key_hist=None, stream=None, bind=False):
    """Top-k of level-two rows whose finite scores lie in the ascending
    candidate blocks cand_blocks [R, n_cand] int32 (the output of
    idx_select_candidate_blocks); scores [R, ld] float32, out [R, ld_out].
    key_hist: the [R, 2048] histogram idx_score produced for these scores
    with these candidate blocks; the call resets it to zero.  Returns k_out."""
    torch = _torch()
    _dev(scores, "scores", (torch.float32,), 2)
    _dev(compress_lens, "compress_lens", (torch.int32,), 1)
    _dev(cand_blocks, "cand_blocks", (torch.int32,), 2)
    _dev(out, "out", (torch.int32,), 2)
    R = scores.shape[0]
    if compress_lens.shape[0] != R or cand_blocks.shape[0] != R or out.shape[0] != R:
        raise ValueError("scores, compress_lens, cand_blocks and out need the same rows")
    if key_hist is not None:
        _dev(key_hist, "key_hist", (torch.int32,), 2)
        if key_hist.shape != (R, 2048):
            raise ValueError("key_hist must be [R, 2048]")
    kout = ctypes.c_int32(-1)
    bound = _issue("idx_topk_candidates", (_ptr(scores), scores.shape[1], R, T,
                                              _ptr(compress_lens), _ptr(cand_blocks),
                                              cand_blocks.shape[1], cand_block_size,
                                              _ptr(key_hist), index_topk, offset, _ptr(out),
                                              out.shape[1], ctypes.byref(kout)), stream,
                   "idx_topk_candidates", bind)
    return bound if bind else kout.value


def idx_select_workspace_size(R, T, ctb, cbs) -> int:
    return int(load_library().idx_select_workspace_size(R, T, ctb, cbs))


def idx_select_candidate_blocks(scores, T, compress_lens, candidate_topk_blocks,
                                cand_block_size, block_ids, workspace=None, stream=None,
                                bind=False):
    torch = _torch()
    _dev(scores, "scores", (torch.float32,), 2)
    _dev(compress_lens, "compress_lens", (torch.int32,), 1)
    _dev(block_ids, "block_ids", (torch.int32,), 2)
    R = scores.shape[0]
    need = idx_select_workspace_size(R, T, candidate_topk_blocks, cand_block_size)
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=scores.device)
    wsb = 0 if workspace is None else workspace.numel() * workspace.element_size()
    return _issue("idx_select_candidate_blocks", (
        _ptr(scores), scores.shape[1], R, T, _ptr(compress_lens), candidate_topk_blocks,
        cand_block_size, _ptr(block_ids), block_ids.shape[1], _ptr(workspace), wsb), stream,
        "idx_select_candidate_blocks", bind, keep=(workspace,))


def idx_publish_keys(latent, wk, gamma, cos_sin, start_pos, ratio, eps, k_cache, rd=64,
                     stream=None, bind=False):
    """latent [B, G, Din] bf16, wk [128, Din] bf16, gamma [128] float32,
    cos_sin [P, rd/2, 2] float32, k_cache [B', Tcap, 68] uint8 (B' >= B)."""
    torch = _torch()
    _dev(latent, "latent", _bf16_types(), 3)
    _dev(wk, "wk", _bf16_types(), 2)
    _dev(gamma, "gamma", (torch.float32,), 1)
    _dev(cos_sin, "cos_sin", (torch.float32,), 3)
    _dev(k_cache, "k_cache", (torch.uint8,), 3)
    B, G, Din = latent.shape
    D = wk.shape[0]
    if wk.shape[1] != Din or gamma.shape[0] != D or k_cache.shape[0] < B:
        raise ValueError("shape mismatch in idx_publish_keys")
    return _issue("idx_publish_keys", (_ptr(latent), _ptr(wk), _ptr(gamma), _ptr(cos_sin),
                                           cos_sin.shape[0], B, G, Din, D, rd, eps, start_pos,
                                           ratio, _ptr(k_cache), k_cache.shape[1],
                                           k_cache.shape[1]), stream, "idx_publish_keys", bind)


def idx_score_topk_candidates(q, w, k_cache, B, S, T, compress_lens, cand_blocks,
                              cand_block_size, slot_scores, index_topk, offset, out,
                              key_hist=None, stream=None, bind=False):
    """The level-two pass: idx_score in candidate mode with the scores kept
    per candidate slot (slot_scores [B*S, ld] float32, ld >= n_cand *
    cand_block_size), then idx_topk_candidates.  Returns k_out (None with
    bind=True)."""
    torch = _torch()
    _dev(q, "q", _bf16_types(), 3)
    _dev(w, "w", _bf16_types(), 2)
    _dev(k_cache, "k_cache", (torch.uint8,), 3)
    _dev(compress_lens, "compress_lens", (torch.int32,), 1)
    _dev(cand_blocks, "cand_blocks", (torch.int32,), 2)
    _dev(slot_scores, "slot_scores", (torch.float32,), 2)
    _dev(out, "out", (torch.int32,), 2)
    R, H, D = q.shape
    if R != B * S or tuple(w.shape) != (R, H) or compress_lens.shape[0] != R:
        raise ValueError("q/w/compress_lens rows must be B*S")
    if k_cache.shape[0] < B or k_cache.shape[2] != ROW_BYTES:
        raise ValueError("k_cache must be [>=B, Tcap, 68]")
    if cand_blocks.shape[0] != R or slot_scores.shape[0] != R or out.shape[0] != R:
        raise ValueError("cand_blocks, slot_scores and out must have B*S rows")
    if key_hist is not None:
        _dev(key_hist, "key_hist", (torch.int32,), 2)
        if tuple(key_hist.shape) != (R, 2048):
            raise ValueError("key_hist must be [B*S, 2048]")
    k = ctypes.c_int32(-1)
    r = _issue("idx_score_topk_candidates",
               (_ptr(q), _ptr(w), _ptr(k_cache), k_cache.shape[1], B, S, H, D, T,
                _ptr(compress_lens), _ptr(cand_blocks), cand_blocks.shape[1], cand_block_size,
                _ptr(slot_scores), slot_scores.shape[1], _ptr(key_hist), index_topk, offset,
                _ptr(out), out.shape[1], ctypes.byref(k)), stream, "idx_score_topk_candidates",
               bind, keep=(k,))
    return r if bind else k.value


def idx_two_level_topk(scores, key_hist, out1, workspace, q, w2, k_cache, B, S, T,
                       compress_lens, cand_blocks, cand_block_size, slot_scores, key_hist2,
                       index_topk, offset, out2, stream=None, bind=False):
    """The rest of a two-level step after the level-one select: idx_topk of
    the level-one scores [B*S, ld] into out1 (key_hist: its histogram,
    workspace: as for idx_topk, allocated here when None), then
    idx_score_topk_candidates with head weights w2 into out2 (slot_scores,
    key_hist2: level two's own buffers).  On the split path the two rankings
    run side by side in one launch."""
    torch = _torch()
    _dev(scores, "scores", (torch.float32,), 2)
    _dev(out1, "out1", (torch.int32,), 2)
    _dev(q, "q", _bf16_types(), 3)
    _dev(w2, "w2", _bf16_types(), 2)
    _dev(k_cache, "k_cache", (torch.uint8,), 3)
    _dev(compress_lens, "compress_lens", (torch.int32,), 1)
    _dev(cand_blocks, "cand_blocks", (torch.int32,), 2)
    _dev(slot_scores, "slot_scores", (torch.float32,), 2)
    _dev(out2, "out2", (torch.int32,), 2)
    R, H, D = q.shape
    if R != B * S or tuple(w2.shape) != (R, H) or compress_lens.shape[0] != R:
        raise ValueError("q/w2/compress_lens rows must be B*S")
    if k_cache.shape[0] < B or k_cache.shape[2] != ROW_BYTES:
        raise ValueError("k_cache must be [>=B, Tcap, 68]")
    for name, t in (("scores", scores), ("out1", out1), ("cand_blocks", cand_blocks),
                    ("slot_scores", slot_scores), ("out2", out2)):
        if t.shape[0] != R:
            raise ValueError(f"{name} must have B*S rows")
    for name, h in (("key_hist", key_hist), ("key_hist2", key_hist2)):
        if h is not None:
            _dev(h, name, (torch.int32,), 2)
            if tuple(h.shape) != (R, 2048):
                raise ValueError(f"{name} must be [B*S, 2048]")
    need = idx_topk_workspace_size(R, T, index_topk)
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=scores.device)
    wsb = 0 if workspace is None else workspace.numel() * workspace.element_size()
    return _issue("idx_two_level_topk",
                  (_ptr(scores), scores.shape[1], _ptr(key_hist), _ptr(out1), out1.shape[1],
                   _ptr(workspace), wsb, _ptr(q), _ptr(w2), _ptr(k_cache), k_cache.shape[1], B, S,
                   H, D, T, _ptr(compress_lens), _ptr(cand_blocks), cand_blocks.shape[1],
                   cand_block_size, _ptr(slot_scores), slot_scores.shape[1], _ptr(key_hist2),
                   index_topk, offset, _ptr(out2), out2.shape[1]), stream, "idx_two_level_topk",
                  bind, keep=(workspace,))


def idx_score_select_blocks(q, w, k_cache, B, S, T, compress_lens, scores, candidate_topk_blocks,
                            cand_block_size, block_ids, workspace, key_hist=None, stream=None,
                            bind=False):
    """idx_score then idx_select_candidate_blocks (the level-one pass):
    arguments as those two wrappers take them; workspace as
    idx_select_workspace_size sizes it."""
    torch = _torch()
    _dev(q, "q", _bf16_types(), 3)
    _dev(w, "w", _bf16_types(), 2)
    _dev(k_cache, "k_cache", (torch.uint8,), 3)
    _dev(compress_lens, "compress_lens", (torch.int32,), 1)
    _dev(scores, "scores", (torch.float32,), 2)
    _dev(block_ids, "block_ids", (torch.int32,), 2)
    _dev(workspace, "workspace", (torch.uint8,), 1)
    R, H, D = q.shape
    if R != B * S or tuple(w.shape) != (R, H) or compress_lens.shape[0] != R:
        raise ValueError("q/w/compress_lens rows must be B*S")
    if k_cache.shape[0] < B or k_cache.shape[2] != ROW_BYTES or scores.shape[0] != R:
        raise ValueError("k_cache must be [>=B, Tcap, 68] and scores [B*S, ld]")
    if block_ids.shape[0] != R:
        raise ValueError("block_ids must have B*S rows")
    if key_hist is not None:
        _dev(key_hist, "key_hist", (torch.int32,), 2)
        if tuple(key_hist.shape) != (R, 2048):
            raise ValueError("key_hist must be [B*S, 2048]")
    return _issue("idx_score_select_blocks",
                  (_ptr(q), _ptr(w), _ptr(k_cache), k_cache.shape[1], B, S, H, D, T,
                   _ptr(compress_lens), _ptr(scores), scores.shape[1], _ptr(key_hist),
                   candidate_topk_blocks, cand_block_size, _ptr(block_ids), block_ids.shape[1],
                   _ptr(workspace), workspace.numel()), stream, "idx_score_select_blocks", bind)


def _publish_score(name, rb, latent, wk, gamma, cos_sin, start_pos, ratio, eps, q, w, k_cache,
                   T, compress_lens, scores, key_hist, rd, stream, bind):
    torch = _torch()
    _dev(latent, "latent", _bf16_types(), 3)
    _dev(wk, "wk", _bf16_types(), 2)
    _dev(gamma, "gamma", (torch.float32,), 1)
    _dev(cos_sin, "cos_sin", (torch.float32,), 3)
    _dev(q, "q", _bf16_types(), 3)
    _dev(w, "w", _bf16_types(), 2)
    _dev(k_cache, "k_cache", (torch.uint8,), 3)
    _dev(compress_lens, "compress_lens", (torch.int32,), 1)
    _dev(scores, "scores", (torch.float32,), 2)
    B, G, Din = latent.shape
    R, H, D = q.shape
    if G != 1 or R != B or tuple(w.shape) != (B, H) or compress_lens.shape[0] != B:
        raise ValueError(f"{name} takes one group and one query row per sequence")
    if wk.shape != (D, Din) or gamma.shape[0] != D or k_cache.shape[0] < B:
        raise ValueError(f"shape mismatch in {name}")
    if k_cache.shape[2] != rb or scores.shape[0] != B:
        raise ValueError(f"k_cache must be [>=B, Tcap, {rb}] and scores [B, ld]")
    if key_hist is not None:
        _dev(key_hist, "key_hist", (torch.int32,), 2)
        if tuple(key_hist.shape) != (B, 2048):
            raise ValueError("key_hist must be [B, 2048]")
    return _issue(name,
                  (_ptr(latent), _ptr(wk), _ptr(gamma), _ptr(cos_sin), cos_sin.shape[0], Din, rd,
                   eps, start_pos, ratio, _ptr(q), _ptr(w), _ptr(k_cache), k_cache.shape[1], B, H,
                   D, T, _ptr(compress_lens), _ptr(scores), scores.shape[1], _ptr(key_hist)),
                  stream, name, bind)


def idx_publish_score(latent, wk, gamma, cos_sin, start_pos, ratio, eps, q, w, k_cache, T,
                      compress_lens, scores, key_hist=None, rd=64, stream=None, bind=False):
    """idx_publish_keys then idx_score for one decode step (one query row and
    one group per sequence): latent [B, 1, Din] bf16, q [B, H, 128] bf16,
    w [B, H] bf16, k_cache [B', Tcap, 68] uint8, compress_lens [B] int32,
    scores [B, ld] float32, key_hist [B, 2048] int32 or None.  One launch
    when the published row is the last scored position (T - 1)."""
    return _publish_score("idx_publish_score", ROW_BYTES, latent, wk, gamma, cos_sin, start_pos,
                          ratio, eps, q, w, k_cache, T, compress_lens, scores, key_hist, rd,
                          stream, bind)


def idx_publish_score_fp8(latent, wk, gamma, cos_sin, start_pos, ratio, eps, q, w, k_cache, T,
                          compress_lens, scores, key_hist=None, rd=64, stream=None, bind=False):
    """idx_publish_keys_fp8 then idx_score_fp8 for one decode step: as
    idx_publish_score, with k_cache [B', Tcap, 132] uint8 FP8 rows."""
    return _publish_score("idx_publish_score_fp8", FP8_ROW_BYTES, latent, wk, gamma, cos_sin,
                          start_pos, ratio, eps, q, w, k_cache, T, compress_lens, scores,
                          key_hist, rd, stream, bind)


def idx_publish_score_paged(latent, wk, gamma, cos_sin, start_pos, ratio, eps, q, w, k_pages,
                            block_table, T, compress_lens, scores, key_hist=None, rd=64,
                            stream=None, bind=False):
    """idx_publish_score on a paged key cache (pages as idx_score_paged):
    latent [B, 1, Din] bf16, q [B, H, 128] bf16, w [B, H] bf16, k_pages
    [n_pages, >=64, 68] uint8, block_table [B, n_blk] int32, compress_lens [B]
    int32, scores [B, ld] float32, key_hist [B, 2048] int32 or None.  One
    launch when the published row is the last scored position (T - 1)."""
    torch = _torch()
    _dev(latent, "latent", _bf16_types(), 3)
    _dev(wk, "wk", _bf16_types(), 2)
    _dev(gamma, "gamma", (torch.float32,), 1)
    _dev(cos_sin, "cos_sin", (torch.float32,), 3)
    _dev(q, "q", _bf16_types(), 3)
    _dev(w, "w", _bf16_types(), 2)
    _dev(compress_lens, "compress_lens", (torch.int32,), 1)
    _dev(scores, "scores", (torch.float32,), 2)
    B, G, Din = latent.shape
    R, H, D = q.shape
    if G != 1 or R != B or tuple(w.shape) != (B, H) or compress_lens.shape[0] != B:
        raise ValueError("idx_publish_score_paged takes one group and one query row per sequence")
    if wk.shape != (D, Din) or gamma.shape[0] != D or scores.shape[0] != B:
        raise ValueError("shape mismatch in idx_publish_score_paged")
    if key_hist is not None:
        _dev(key_hist, "key_hist", (torch.int32,), 2)
        if tuple(key_hist.shape) != (B, 2048):
            raise ValueError("key_hist must be [B, 2048]")
    ps, npg, bts = _pages(k_pages, block_table, B)
    return _issue("idx_publish_score_paged",
                  (_ptr(latent), _ptr(wk), _ptr(gamma), _ptr(cos_sin), cos_sin.shape[0], Din, rd,
                   eps, start_pos, ratio, _ptr(q), _ptr(w), _ptr(k_pages), ps, npg,
                   _ptr(block_table), bts, B, H, D, T, _ptr(compress_lens), _ptr(scores),
                   scores.shape[1], _ptr(key_hist)),
                  stream, "idx_publish_score_paged", bind)


def idx_yarn_cos_sin(P, rd, theta, factor, orig_len, beta_fast, beta_slow):
    """Host table [P, rd/2, 2] float32 (numpy) for idx_publish_keys."""
    import numpy as np
    out = np.empty((P, rd // 2, 2), np.float32)
    _check(load_library().idx_yarn_cos_sin(P, rd, theta, factor, orig_len, beta_fast, beta_slow,
                                           out.ctypes.data_as(ctypes.c_void_p)),
           "idx_yarn_cos_sin")
    return out


def idx_timing_arm(slot: int):
    """Time the next score launch (idx_score / idx_score_topk) into event pair `slot`."""
    _check(load_library().idx_timing_arm(int(slot)), "idx_timing_arm")


def idx_timing_read(slot: int) -> float:
    """Duration in ms of the score kernel timed into `slot` (waits for it)."""
    ms = ctypes.c_float()
    _check(load_library().idx_timing_read(int(slot), ctypes.byref(ms)), "idx_timing_read")
    return float(ms.value)


def idx_probe_stream_read(buf, grid, sink, stream=None) -> float:
    """Measured streaming read of the whole device tensor `buf` (its bytes a
    multiple of 16) by `grid` workgroups; sink: int32 device tensor of at
    least `grid` words.  Returns the kernel's duration in ms (waits)."""
    nbytes = buf.numel() * buf.element_size()
    if sink.numel() < grid:
        raise ValueError("sink needs a word per workgroup")
    ms = ctypes.c_float()
    _check(load_library().idx_probe_stream_read(_ptr(buf), nbytes, grid, _ptr(sink),
                                                ctypes.byref(ms), _stream(stream)),
           "idx_probe_stream_read")
    return float(ms.value)


def idx_probe_mfma_fp4(grid, iters, sink, stream=None):
    """Measured fp4 matrix-core loop: returns (flops, ms).  sink: float32
    device tensor of at least grid * 256 elements."""
    if sink.numel() < grid * 256:
        raise ValueError("sink needs grid * 256 floats")
    ms, fl = ctypes.c_float(), ctypes.c_double()
    _check(load_library().idx_probe_mfma_fp4(grid, iters, _ptr(sink), ctypes.byref(fl),
                                             ctypes.byref(ms), _stream(stream)),
           "idx_probe_mfma_fp4")
    return float(fl.value), float(ms.value)


def idx_probe_bf16_convert(stream=None) -> int:
    """The number of finite fp32 inputs on which the bf16 conversion
    instruction differs from the software round-to-nearest-even (0 expected)."""
    torch = _torch()
    count = torch.zeros(1, dtype=torch.int64, device="cuda")
    n = ctypes.c_ulonglong(0)
    _check(load_library().idx_probe_bf16_convert(_ptr(count), ctypes.byref(n), _stream(stream)),
           "idx_probe_bf16_convert")
    return int(n.value)
