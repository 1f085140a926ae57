#!/usr/bin/env python3
"""Benchmark of the DeepSeek-V4.1 Indexer hot path on one MI355X.

One step = one pass of the hot path over one batch of synthetic input:
[key publish] -> fp4 score (in-kernel q quantisation, scaled-fp4 MFMA,
fixed-order head sum, causal mask) -> [block select -> level-one top-k ->
level-two score] -> top-k in position order.  The default workload is the
batched decode at 128K tokens (batch 64, 32768 compressed keys per
sequence, 64 heads x 128, top-2048), on which the metric is quoted.

Inputs are seeded synthetic tensors (no dataset), generated on the host,
uploaded once and resident in HBM before timing.  The key cache is kept in
several copies that consecutive steps cycle through, so keys stream from HBM
rather than from the 256 MB last-level cache.

Prints one JSON line (rank 0, N = 1):
  value         queries/s over the K timed steps (host clock, synchronised)
  roofline      the score kernel: algorithmic bytes per launch / its mean
                duration from a HIP event pair attached to each launch on
                the launch stream (hipExtLaunchKernel), against 8 TB/s
  cpu_baseline  the CPU oracle timed on the host on a bounded sample
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = ("indexer queries/sec + keys scored/sec (decode, 128K ctx); % HBM / MFMA roofline")
HBM_PEAK_GBS = 8000.0
FP4_PEAK_TFLOPS = 10100.0
LLC_BYTES = 256 * 2 ** 20


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", type=int, default=1, help="workload id 0..4 (1 = batched decode)")
    ap.add_argument("--event-every", type=int, default=25,
                    help="time the score launch with HIP events on every n-th step of the "
                         "timed region (a timed launch costs the host about 20 us)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="minimum CPU work for the oracle baseline sample")
    ap.add_argument("--paged", action="store_true",
                    help="key cache in pages of 64 positions behind a block table (the paged "
                         "entry points)")
    ap.add_argument("--q-step", action="store_true",
                    help="start from the query heads before RoPE: the step first runs the "
                         "query step (RoPE, fp4 quantise, weight scaling)")
    ap.add_argument("--prefill-publish", action="store_true",
                    help="prefill workloads: the step first publishes the S / ratio keys of "
                         "the prompt (key publish of many groups)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 256 MiB device copy (for counter calibration)")
    return ap.parse_args()


def scored_compress_lens(wl, st):
    """compress_lens of the rows the score launch scores: every row, except
    that the fused launch without scores kept writes rows whose compress_lens
    is at most k_out in closed form, without scoring them."""
    import numpy as np
    cl = np.minimum(wl.compress_lens().astype(np.int64), wl.T)
    if st.fused and st.scores is None:
        cl = np.where(cl > min(wl.topk, wl.T), cl, 0)
    return cl


def score_kernel_bytes(wl, st) -> int:
    """Algorithmic HBM bytes of one score launch: per scored (row, key) pair
    the 68-byte key row and the 4-byte fp32 score; per row the bf16 query
    (H x 128 x 2) and the bf16 weights (H x 2)."""
    cl = scored_compress_lens(wl, st)
    pairs = int(cl.sum())
    rows = int((cl > 0).sum())
    return pairs * (68 + 4) + rows * (wl.H * 128 * 2 + wl.H * 2)


def score_kernel_flops(wl, st) -> int:
    return int(scored_compress_lens(wl, st).sum()) * wl.H * 128 * 2


def score_kernel_name(st) -> str:
    """The launch the score events bracket: the fused score + top-k kernel for
    single-level rows up to 8192 positions, else the score kernel."""
    if st.fused:
        return "idx::score_kernel<2, false, true> (score and top-k in one launch)"
    return "idx::score_kernel<2, false, false>"


def source_digest() -> str:
    h = hashlib.sha256()
    for name in ("score.hip", "idx_common.hpp", "row_topk.hpp"):
        with open(os.path.join(ROOT, "sparse_attention_top_fp4_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(wl_name):
    """HBM bytes per score launch from the committed counter summary, or None
    when absent or taken on a different kernel source."""
    path = os.path.join(ROOT, "profiles", "score_kernel_traffic.json")
    try:
        with open(path) as f:
            d = json.load(f)
    except OSError:
        return None
    e = d.get(wl_name)
    if not e or e.get("source_digest") != source_digest():
        return None
    return e.get("bytes_per_launch")


def cpu_baseline(wl, inp, min_seconds):
    """The oracle as it stands, on the host, on the same workload: quantise q,
    score every reachable key, top-k (the key cache is an input and is
    quantised outside the timed region).  Repeats the sample until at least
    min_seconds of CPU work."""
    import ctypes

    import numpy as np

    import oracle
    kc, _ = oracle.fp4_quant_rows(inp["k"])
    lib = oracle.lib()
    try:
        threads = int(ctypes.CDLL("libgomp.so.1").omp_get_max_threads())
    except OSError:
        threads = os.cpu_count()
    reps, t0 = 0, time.perf_counter()
    while True:
        s, _ = oracle.score(inp["q"], inp["w"], kc, wl.B, wl.S, wl.H, wl.T, inp["cl"])
        if wl.ctb:
            ids = oracle.select_blocks(s, inp["cl"], wl.ctb, wl.cbs)
            oracle.topk(s, inp["cl"], wl.topk, wl.offset)
            s, _ = oracle.score(inp["q"], inp["w2"], kc, wl.B, wl.S, wl.H, wl.T, inp["cl"],
                                cand=ids, cbs=wl.cbs)
        oracle.topk(s, inp["cl"], wl.topk, wl.offset)
        reps += 1
        el = time.perf_counter() - t0
        if el >= min_seconds:
            break
    del lib
    return {"value": reps * wl.R / el, "unit": "queries/s", "cores": threads, "kind": "oracle",
            "sample": f"{reps} full step(s) of {wl.name} ({wl.R} queries x {wl.T} keys), "
                      f"{el:.1f} s"}


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    import sparse_attention_top_fp4_amd as idx
    from sparse_attention_top_fp4_amd.inputs import generate, workload
    from sparse_attention_top_fp4_amd.pipeline import IndexerStep

    idx.load_library()
    wl = workload(args.config)
    t_gen = time.perf_counter()
    inp = generate(wl)
    t_gen = time.perf_counter() - t_gen
    cache_bytes = wl.B * wl.T * 68
    n_caches = max(1, min(8, math.ceil(3 * LLC_BYTES / cache_bytes))) if cache_bytes > 2 ** 20 else 1
    # the product path: indices only (a fused launch does not write scores)
    publish = None
    if args.prefill_publish:
        if wl.start_pos != 0 or wl.S < wl.ratio:
            sys.exit("--prefill-publish needs a prefill workload")
        from sparse_attention_top_fp4_amd.inputs import publish_inputs
        inp.update(publish_inputs(wl, wl.S // wl.ratio, wl.seed() + 1000))
        publish = True
    st = IndexerStep(wl, inp, n_caches=n_caches, keep_scores=False, paged=args.paged,
                     q_step=args.q_step, publish=publish)
    torch.cuda.synchronize()

    for _ in range(args.warmup):
        st.step()
    torch.cuda.synchronize()

    # the score launch of every n-th step of the timed region is timed by a
    # HIP event pair that the library attaches to the launch itself
    # (hipExtLaunchKernel on the launch stream: the kernel's own start and
    # end, no marker packets between the kernels of a step)
    every = max(1, args.event_every)
    timed = list(range(0, args.steps, every))[:256]
    slot = {i: n for n, i in enumerate(timed)}
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        st.step(time_slot=slot.get(i))
    torch.cuda.synchronize()
    t1 = time.perf_counter()

    if args.copy_calibration:
        # known-size reference kernels for the counter calibration: a 256 MiB
        # device copy and an elementwise negation that reads and writes 256 MiB
        a = torch.ones(64 * 2 ** 20, dtype=torch.float32, device="cuda")
        b = torch.empty_like(a)
        b.copy_(a)
        torch.neg(a, out=b)
        torch.cuda.synchronize()

    step_s = (t1 - t0) / args.steps
    score_ms = float(np.mean([idx.idx_timing_read(n) for n in slot.values()]))
    kb = score_kernel_bytes(wl, st)
    kf = score_kernel_flops(wl, st)
    prefill = wl.S > 1
    if prefill:  # many queries share each key: the contraction bounds the kernel
        roof = {"bound": "mfma", "achieved": kf / (score_ms * 1e-3) / 1e12,
                "peak": FP4_PEAK_TFLOPS, "unit": "TFLOP/s"}
    else:
        roof = {"bound": "hbm", "achieved": kb / (score_ms * 1e-3) / 1e9, "peak": HBM_PEAK_GBS,
                "unit": "GB/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    qps = wl.R / step_s
    keys = st.keys_scored()
    # the committed counter summary covers the contiguous layout
    traffic = None if args.paged else measured_traffic(wl.name)
    line = {
        "metric": METRIC,
        "value": qps,
        "unit": "queries/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": step_s * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp4xfp4->f32",
        "data": "synthetic",
        "config": {"workload": wl.name, "batch": wl.B, "queries_per_seq": wl.S,
                   "end_pos": wl.end_pos, "compress_ratio": wl.ratio, "compressed_keys": wl.T,
                   "index_n_heads": wl.H, "index_head_dim": 128, "index_topk": wl.topk,
                   "candidate_topk_blocks": wl.ctb, "candidate_block_size": wl.cbs,
                   "publish": wl.publish, "key_cache_copies": n_caches,
                   "key_cache_layout": "paged" if args.paged else "contiguous",
                   "query_step": bool(args.q_step),
                   "prefill_publish": bool(args.prefill_publish)},
        "keys_scored_per_s": keys / step_s,
        "score_kernel_ms": score_ms,
        "score_kernel_timed_steps": len(timed),
        "roofline": dict(roof, traffic=traffic, kernel=score_kernel_name(st),
                         algorithmic_bytes_per_launch=kb, algorithmic_flops_per_launch=kf),
    }
    if not args.no_cpu:
        line["cpu_baseline"] = cpu_baseline(wl, inp, args.cpu_seconds)
    else:
        line["cpu_baseline"] = None
    print(json.dumps(line), flush=True)
    del t_gen


if __name__ == "__main__":
    main()
