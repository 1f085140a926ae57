"""idx_topk_noalloc, the allocation-free top-k, called through the C ABI
against idx_topk with a caller workspace on the same inputs: the indices
must be identical (bit-exact) and equal to the oracle's top-k, on two calls
in a row, the second with a smaller input, for the paths that take a
workspace (split rows over two kernels, the chunked path).  Sizes beyond
the static workspace are refused before any launch."""
import ctypes

import numpy as np
import pytest

import oracle

from gpu_util import dev, host, say, sync, torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def idx():
    import sparse_attention_top_fp4_amd as m
    L = m.load_library()
    P, i32, i64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64
    L.idx_topk_noalloc.argtypes = [P, i64, i32, i32, P, P, i32, ctypes.c_int32, P, i64, P, P]
    L.idx_topk_noalloc.restype = i32
    L.idx_topk_noalloc_max_workspace.restype = ctypes.c_size_t
    return m


def _host_hist(scores, cl):
    """Top-11-bit order-key counts of each row's positions below cl."""
    out = np.zeros((scores.shape[0], 2048), np.int32)
    for r in range(scores.shape[0]):
        v = scores[r, :cl[r]].astype(np.float32)
        v = np.where(v == 0.0, np.float32(0.0), v)
        u = v.view(np.uint32)
        key = np.where(u & 0x80000000, ~u, u | 0x80000000).astype(np.uint32)
        out[r] = np.bincount(key >> 21, minlength=2048)
    return out


def _case(seed, R, T):
    rng = np.random.default_rng(seed)
    s = rng.standard_normal((R, T)).astype(np.float32)
    s[:, ::7] = np.round(s[:, ::7], 1)  # ties
    cl = np.full(R, T, np.int32)
    cl[0] = T - 17
    return s, cl


# (R, T, path) pairs: each call followed by a smaller one
CALLS = [
    [(4, 65536, "auto"), (2, 40000, "auto")],       # split rows
    [(3, 9000, "chunked"), (1, 5000, "chunked")],   # chunked path
]


@pytest.mark.parametrize("calls", CALLS)
def test_noalloc_topk_matches_topk(idx, calls, monkeypatch):
    t = torch()
    L = idx.load_library()
    k, offset = 2048, 5
    for n, (R, T, path) in enumerate(calls):
        if path == "chunked":
            monkeypatch.setenv("IDX_TOPK_PATH", "chunked")
        say("noalloc top-k", n, R, T, path)
        s, cl = _case(100 + n + T, R, T)
        h = _host_hist(s, cl)
        sd, cld = dev(s), dev(cl)
        kout = min(k, T)
        out_ref = t.full((R, kout), -7, dtype=t.int32, device="cuda")
        got = idx.idx_topk(sd, T, cld, k, offset, out_ref, key_hist=dev(h))
        assert got == kout
        out = t.full((R, kout), -9, dtype=t.int32, device="cuda")
        hist = dev(h)
        ko = ctypes.c_int32(-1)
        stream = ctypes.c_void_p(t.cuda.current_stream().cuda_stream)
        st = L.idx_topk_noalloc(ctypes.c_void_p(sd.data_ptr()), T, R, T,
                                ctypes.c_void_p(cld.data_ptr()), ctypes.c_void_p(hist.data_ptr()),
                                k, offset, ctypes.c_void_p(out.data_ptr()), kout,
                                ctypes.byref(ko), stream)
        assert st == 0 and ko.value == kout
        sync()
        assert np.array_equal(host(out), host(out_ref))
        assert np.array_equal(host(out), oracle.topk(s, cl, k, offset))
        assert not host(hist).any()


def test_noalloc_refuses_oversized_workspace(idx):
    L = idx.load_library()
    assert L.idx_topk_noalloc_max_workspace() == 16 << 20
    d = ctypes.c_void_p(0x1000)
    # 8 rows of 262144 positions need more than 16 MiB of split workspace
    assert L.idx_topk_noalloc(d, 262144, 8, 262144, d, d, 2048, 0, d, 2048, None, None) == 2
    assert L.idx_topk_noalloc(d, 262144, 7, 262144, d, None, 0, 0, d, 2048, None, None) == 1
