"""Calls from several host threads: two threads, each with its own stream
(default priority) and buffers, issue score + histogram + top-k and the
fused score + top-k concurrently; every iteration's indices and scores must
equal the oracle's.  (ctypes releases the interpreter lock around each
call, so the launches do interleave.)"""
import threading

import numpy as np
import pytest

import oracle
from sparse_attention_top_fp4_amd.inputs import small_case

from gpu_util import bits, dev, fp4_cache, host, say, sync, torch

pytestmark = pytest.mark.gpu


def test_two_threads_two_streams():
    import sparse_attention_top_fp4_amd as idx
    idx.load_library()
    t = torch()
    B, S, H, T, k, off = 2, 3, 64, 3000, 700, 11
    say("threads", B, S, H, T, k)
    c = small_case(131, B, S, H, T, start_pos=4000)
    R = B * S
    kc_ref, _ = oracle.fp4_quant_rows(c["k"])
    ref, _ = oracle.score(c["q"], c["w"], kc_ref, B, S, H, T, c["cl"])
    ref_idx = oracle.topk(ref, c["cl"], k, off)
    kc = fp4_cache(c["k"])
    q, w, cl = dev(c["q"]), dev(c["w"]), dev(c["cl"])
    n_iter = 25

    class Worker:
        def __init__(self):
            self.stream = t.cuda.Stream()
            self.sc = t.empty((R, T), dtype=t.float32, device="cuda")
            self.hist = t.empty((R, 2048), dtype=t.int32, device="cuda")
            self.ws = t.empty(max(idx.idx_topk_workspace_size(R, T, k), 1), dtype=t.uint8,
                              device="cuda")
            self.out = t.empty((n_iter, R, k), dtype=t.int32, device="cuda")
            self.out_f = t.empty((n_iter, R, k), dtype=t.int32, device="cuda")
            self.sc_keep = t.empty((n_iter, R, T), dtype=t.float32, device="cuda")
            self.err = None
            idx.idx_clear_key_hist(self.hist, stream=self.stream)

        def run(self):
            try:
                for i in range(n_iter):
                    idx.idx_score(q, w, kc, B, S, T, cl, self.sc, key_hist=self.hist,
                                  stream=self.stream)
                    idx.idx_topk(self.sc, T, cl, k, off, self.out[i], workspace=self.ws,
                                 key_hist=self.hist, stream=self.stream)
                    idx.idx_score_topk(q, w, kc, B, S, T, cl, k, off, self.out_f[i],
                                       scores=self.sc_keep[i], stream=self.stream)
            except Exception as e:  # reported on the main thread
                self.err = e

    sync()
    workers = [Worker(), Worker()]
    sync()
    threads = [threading.Thread(target=wk.run) for wk in workers]
    for th in threads:
        th.start()
    for th in threads:
        th.join()
    sync()
    for wk in workers:
        assert wk.err is None, wk.err
        out, out_f, sk = host(wk.out), host(wk.out_f), host(wk.sc_keep)
        for i in range(n_iter):
            assert np.array_equal(out[i], ref_idx), ("score+topk", i)
            assert np.array_equal(out_f[i], ref_idx), ("fused", i)
        for r in range(R):
            n = int(c["cl"][r])
            assert np.array_equal(bits(sk[:, r, :n]), np.broadcast_to(bits(ref[r, :n]),
                                                                        (n_iter, n))), r
