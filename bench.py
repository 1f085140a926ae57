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
  roofline      the score kernel: algorithmic bytes (decode: keys, fp4 query
                heads, weights) or fp4 flops (prefill: every causal pair)
                per launch / its mean duration from HIP event pairs attached
                to eight launches of the timed region on the launch
                stream (hipExtLaunchKernel), against 8 TB/s or 10.1 PFLOP/s;
                roofline.step: the whole step's algorithmic bytes or flops
                over ms_per_step against the same peak
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
FP8_PEAK_TFLOPS = 5000.0
LLC_BYTES = 256 * 2 ** 20


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", type=int, default=1, help="workload id 0..4 (1 = batched decode)")
    ap.add_argument("--event-every", type=int, default=0,
                    help="time the score launch with HIP events on every n-th step of the "
                         "timed region; 0 (default): eight steps spread over it (a timed "
                         "launch costs the host about 30 us)")
    ap.add_argument("--latency-steps", type=int, default=50,
                    help="after the timed region, this many single steps each bracketed by "
                         "an event pair, for the p10/p50/p90 step time")
    ap.add_argument("--cpu-threads", type=int, default=0,
                    help="OpenMP threads of the oracle baseline (0: all host cores)")
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
    ap.add_argument("--fp8", action="store_true",
                    help="key cache in FP8 rows (132 bytes: 128 e4m3 codes + fp32 scale per "
                         "128 values), scored on the e4m3 matrix core")
    ap.add_argument("--ceilings", action="store_true",
                    help="only measure the chip's ceilings (streaming read over grid sizes, "
                         "fp4 matrix-core loop) and print them as one JSON line")
    ap.add_argument("--tsplit", type=int, default=0,
                    help="only measure one owner's share of the ranking when the rows are "
                         "split along their positions over this many owners (the top-k of "
                         "one slice as (position, score) pairs and the merge of every "
                         "slice's list) and print it as one JSON line")
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


Q_ROW_BYTES = 68       # one fp4 query head: 64 code bytes + 4 scale bytes
FLOP_PER_PAIR_HEAD = 2 * 128


def reachable_pairs(wl) -> int:
    """(row, key) pairs below compress_lens: the causal pairs of a prefill,
    B * T for a decode."""
    import numpy as np
    return int(np.minimum(wl.compress_lens().astype(np.int64), wl.T).sum())


def publish_bytes(wl, groups=1, rb=68) -> int:
    """The key publish: wk once, each group's bf16 latent and its written row."""
    return 128 * wl.din * 2 + wl.B * groups * (wl.din * 2 + rb)


def score_kernel_bytes(wl, st=None, rb=68, publish=False) -> int:
    """Algorithmic HBM bytes of one (level-one) score launch: the key row
    (rb bytes: 68 fp4, 132 FP8) of every reachable (row, key) pair, each
    row's quantised query heads (rb bytes a head) and its bf16 weights, and
    with `publish` the decode key publish the launch also runs.  The fp32
    score scratch the launch also writes is an implementation cost, not
    algorithmic: it shows up in the measured traffic instead."""
    b = reachable_pairs(wl) * rb + wl.R * wl.H * (rb + 2)
    return b + (publish_bytes(wl, 1, rb) if publish else 0)


def score_kernel_flops(wl, st=None) -> int:
    """Algorithmic fp4 flops of one score launch: 2 * 128 per head for every
    reachable pair.  A prefill's rows with compress_lens <= k_out are part of
    it even where the fused launch writes them in closed form."""
    return reachable_pairs(wl) * wl.H * FLOP_PER_PAIR_HEAD


def scored_flops(wl, st) -> int:
    """The flops the launch actually performs (closed-form rows excluded)."""
    return int(scored_compress_lens(wl, st).sum()) * wl.H * FLOP_PER_PAIR_HEAD


def step_bytes(wl, q_step=False, prefill_publish_groups=0, rb=68) -> int:
    """Algorithmic HBM bytes of one whole step: every score launch's keys,
    the quantised query and the weights (per level), the candidate block
    ids, the key publish (wk, latent, the written rows) and the int32
    indices of every top-k the step keeps.  rb: bytes of a key row."""
    kout = min(wl.topk, wl.T)
    b = reachable_pairs(wl) * rb + wl.R * wl.H * (rb + 2) + wl.R * kout * 4
    if wl.ctb:
        nb = -(-wl.T // wl.cbs)
        cand = wl.R * min(wl.ctb * wl.cbs, wl.T)
        b += cand * rb + wl.R * wl.H * 2            # level-two keys and weights
        b += wl.R * min(wl.ctb, nb) * 4              # block ids
        b += wl.R * kout * 4                         # level-one indices
    if wl.publish:
        b += publish_bytes(wl, 1, rb)
    if q_step:
        # the step starts from the bf16 heads before RoPE and the raw weights;
        # the quantised heads and scaled weights are intermediate
        b += wl.R * wl.H * (128 * 2 + 2) - wl.R * wl.H * (rb + 2)
    if prefill_publish_groups:
        b += publish_bytes(wl, prefill_publish_groups, 68)
    return b


def step_flops(wl) -> int:
    f = score_kernel_flops(wl)
    if wl.ctb:
        f += wl.R * min(wl.ctb * wl.cbs, wl.T) * wl.H * FLOP_PER_PAIR_HEAD
    return f


def percentiles(xs):
    import numpy as np
    a = np.asarray(xs, dtype=np.float64)
    return {"p10": float(np.percentile(a, 10)), "p50": float(np.percentile(a, 50)),
            "p90": float(np.percentile(a, 90)), "mean": float(a.mean()), "n": int(a.size)}


def timed_steps(steps: int, target: int = 8):
    """Steps of the timed region whose score launch is timed: `target` of
    them (all steps when fewer), spread evenly over the region and not
    starting at its first step.  A timed launch costs the host about 30 us,
    so timing fewer launches disturbs the region less."""
    if steps <= target:
        return list(range(steps))
    return sorted({int(round((i + 0.5) * steps / target)) for i in range(target)})


def score_kernel_name(st) -> str:
    """The launch the score events bracket: the fused score + top-k kernel for
    single-level rows up to 8192 positions, else the score kernel."""
    if st.fused:
        return "idx::score_kernel<2, false, true, false> (score and top-k in one launch)"
    if getattr(st, "fp8", False):
        return "idx::score_kernel<2, false, false, true> (FP8 rows)"
    if getattr(st, "publish_in_score", False):
        return "idx::score_kernel<2, false, false, false> (with the key publish workgroups)"
    if getattr(st, "two_level", False):
        return "idx::score_kernel<2, false, false, false> (level one, with its block maxima)"
    return "idx::score_kernel<2, false, false, false>"


def source_digest() -> str:
    h = hashlib.sha256()
    for name in ("score.hip", "idx_common.hpp", "row_topk.hpp", "publish_dev.hpp", "split_topk.hpp"):
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


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(wl, inp, min_seconds, threads=None):
    """The oracle as it stands, on the host, on the same workload: quantise q,
    score every reachable key, top-k (the key cache is an input and is
    quantised outside the timed region).  Repeats the sample until at least
    min_seconds of CPU work.  threads: OpenMP thread count (default: all)."""
    import ctypes

    import numpy as np

    import oracle
    kc, _ = oracle.fp4_quant_rows(inp["k"])
    lib = oracle.lib()
    try:
        gomp = ctypes.CDLL("libgomp.so.1")
        if threads:
            gomp.omp_set_num_threads(int(threads))
        threads = int(gomp.omp_get_max_threads())
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
            "cpu_model": cpu_model(), "host_cpus": os.cpu_count(),
            "sample": f"{reps} full step(s) of {wl.name} ({wl.R} queries x {wl.T} keys), "
                      f"{el:.1f} s"}


STREAM_GRIDS = (256, 512, 1024, 2048, 4096)


def measure_ceilings(nbytes, reps=8):
    """Streaming-read ceiling over `nbytes` (read from several copies in
    turn, so the 256 MB last-level cache does not serve them) for each grid
    size, and the fp4 matrix-core ceiling.  Best and median of `reps`."""
    import numpy as np
    import torch

    import sparse_attention_top_fp4_amd as idx
    n = -(-nbytes // 16) * 4  # int32 words, a multiple of 16 bytes
    copies = max(2, math.ceil(3 * LLC_BYTES / (n * 4)))
    bufs = [torch.ones(n, dtype=torch.int32, device="cuda") for _ in range(copies)]
    sink = torch.empty(max(STREAM_GRIDS) * 256, dtype=torch.int32, device="cuda")
    stream = {}
    for g in STREAM_GRIDS:
        ms = [idx.idx_probe_stream_read(bufs[i % copies], g, sink) for i in range(reps + 1)][1:]
        gbs = [n * 4 / (m * 1e-3) / 1e9 for m in ms]
        stream[str(g)] = {"best_GBs": max(gbs), "median_GBs": float(np.median(gbs))}
    best = max(stream.values(), key=lambda v: v["best_GBs"])
    del bufs
    fsink = torch.empty(512 * 256, dtype=torch.float32, device="cuda")
    mf = []
    for g in (256, 512):
        runs = [idx.idx_probe_mfma_fp4(g, 4000, fsink) for _ in range(4)][1:]
        mf.append({"grid": g, "best_TFLOPs": max(f / (m * 1e-3) / 1e12 for f, m in runs)})
    return {"stream_read": {"bytes": n * 4, "copies": copies, "by_grid": stream,
                            "best_GBs": best["best_GBs"], "median_GBs": best["median_GBs"]},
            "mfma_fp4": {"by_grid": mf, "best_TFLOPs": max(m["best_TFLOPs"] for m in mf)}}


def measure_tsplit(wl, G, steps, warmup):
    """One owner's share of the ranking of a T-split: the rows' positions in
    G equal slices, each owner ranking its slice (idx_topk_pairs, here the
    last slice, without a score histogram) and every owner merging the G
    gathered lists (idx_merge_topk).  The scores are one step's of the
    workload on one GPU; the merged rows are checked against idx_topk of the
    whole rows before timing.  Times are event pairs around `steps` calls."""
    import torch

    import sparse_attention_top_fp4_amd as idx
    from sparse_attention_top_fp4_amd.inputs import generate
    from sparse_attention_top_fp4_amd.pipeline import IndexerStep

    R, T, k = wl.R, wl.T, wl.topk
    if G < 2 or T % G:
        sys.exit(f"--tsplit {G}: needs at least 2 slices that divide T = {T}")
    st = IndexerStep(wl, generate(wl))
    st.step()
    torch.cuda.synchronize()
    Tg = T // G
    n = min(k, Tg)
    kout = min(k, T)
    pos = torch.full((G, R, n), -1, dtype=torch.int32, device="cuda")
    sco = torch.full((G, R, n), float("-inf"), dtype=torch.float32, device="cuda")
    ws = torch.empty(max(1, idx.idx_topk_pairs_workspace_size(R, Tg, k)), dtype=torch.uint8,
                     device="cuda")
    for g in range(G):
        idx.idx_topk_pairs(st.scores, g * Tg, Tg, st.cl, k, pos[g], sco[g], workspace=ws)
    out = torch.empty((R, kout), dtype=torch.int32, device="cuda")
    idx.idx_merge_topk(pos, sco, st.cl, T, k, wl.offset, out)
    whole = torch.empty((R, kout), dtype=torch.int32, device="cuda")
    idx.idx_topk(st.scores, T, st.cl, k, wl.offset, whole)
    torch.cuda.synchronize()
    if not torch.equal(out, whole):
        sys.exit("--tsplit: the merged rows differ from the whole rows' top-k")
    g = G - 1
    pairs = idx.idx_topk_pairs(st.scores, g * Tg, Tg, st.cl, k, pos[g], sco[g], workspace=ws,
                               bind=True)
    merge = idx.idx_merge_topk(pos, sco, st.cl, T, k, wl.offset, out, bind=True)

    def timed(calls):
        for _ in range(warmup):
            for c in calls:
                c()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record()
        for _ in range(steps):
            for c in calls:
                c()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) * 1e3 / steps

    pairs_us, merge_us, share_us = timed([pairs]), timed([merge]), timed([pairs, merge])
    return {"metric": "T-split ranking share per owner (us)", "value": share_us, "unit": "us",
            "higher_is_better": False, "steps": steps, "warmup": warmup,
            "config": {"workload": wl.name, "rows": R, "positions": T, "slices": G,
                       "slice_positions": Tg, "index_topk": k, "pairs_per_list": n},
            "pairs_us": pairs_us, "merge_us": merge_us, "share_us": share_us,
            "exchange_bytes": G * R * n * 8,
            "checked": "merged rows equal idx_topk of the whole rows"}


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
    if args.ceilings:
        print(json.dumps({"ceilings": measure_ceilings(wl.B * wl.T * 68),
                          "workload_bytes_from": wl.name}), flush=True)
        return
    if args.tsplit:
        print(json.dumps(measure_tsplit(wl, args.tsplit, args.steps, args.warmup)), flush=True)
        return
    t_gen = time.perf_counter()
    inp = generate(wl)
    t_gen = time.perf_counter() - t_gen
    rb = 132 if args.fp8 else 68
    cache_bytes = wl.B * wl.T * rb
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
                     q_step=args.q_step, publish=publish, fp8=args.fp8)
    torch.cuda.synchronize()

    timed = (timed_steps(args.steps) if args.event_every <= 0
             else list(range(0, args.steps, args.event_every))[:256])
    slot = {i: n for n, i in enumerate(timed)}
    # the warm-up also times one launch into every event pair, so the pairs
    # exist before the timed region (creating one costs the host more than a
    # step)
    for i in range(max(args.warmup, len(timed))):
        st.step(time_slot=i if i < len(timed) else None)
    torch.cuda.synchronize()

    # the score launch of eight steps spread over the timed region is timed
    # by a HIP event pair that the library attaches to the launch itself
    # (hipExtLaunchKernel on the launch stream: the kernel's own start and
    # end, no marker packets between the kernels of a step)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        st.step(time_slot=slot.get(i))
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    score_ms_all = [idx.idx_timing_read(n) for n in slot.values()]

    # after the timed region: the distribution of single-step times, each
    # step bracketed by an event pair on the stream the steps run on
    lat_us = []
    if args.latency_steps > 0:
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(args.latency_steps)]
        for a, b in ev:
            a.record()
            st.step()
            b.record()
        torch.cuda.synchronize()
        lat_us = [a.elapsed_time(b) * 1e3 for a, b in ev]

    if args.copy_calibration:
        # known-size reference kernels for the counter calibration: a 256 MiB
        # device copy and an elementwise negation that reads and writes 256 MiB
        a = torch.ones(64 * 2 ** 20, dtype=torch.float32, device="cuda")
        b = torch.empty_like(a)
        b.copy_(a)
        torch.neg(a, out=b)
        torch.cuda.synchronize()

    step_s = (t1 - t0) / args.steps
    score_ms = float(np.mean(score_ms_all))
    kb = score_kernel_bytes(wl, rb=rb, publish=getattr(st, "publish_in_score", False))
    kf = score_kernel_flops(wl)
    groups = wl.S // wl.ratio if args.prefill_publish else 0
    sb = step_bytes(wl, q_step=args.q_step, prefill_publish_groups=groups, rb=rb)
    sf = step_flops(wl)
    prefill = wl.S > 1
    if prefill:  # many queries share each key: the contraction bounds the kernel
        roof = {"bound": "mfma", "achieved": kf / (score_ms * 1e-3) / 1e12,
                "peak": FP8_PEAK_TFLOPS if args.fp8 else FP4_PEAK_TFLOPS, "unit": "TFLOP/s"}
        step_roof = {"achieved": sf / step_s / 1e12, "flops": sf}
    else:
        roof = {"bound": "hbm", "achieved": kb / (score_ms * 1e-3) / 1e9, "peak": HBM_PEAK_GBS,
                "unit": "GB/s"}
        step_roof = {"achieved": sb / step_s / 1e9, "bytes": sb}
    roof["frac"] = roof["achieved"] / roof["peak"]
    step_roof["frac"] = step_roof["achieved"] / roof["peak"]
    qps = wl.R / step_s
    keys = st.keys_scored()
    # the committed counter summary covers the contiguous layout
    traffic = None if (args.paged or args.fp8 or args.q_step) else measured_traffic(wl.name)
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
        "dtype": "fp8xfp8->f32" if args.fp8 else "fp4xfp4->f32",
        "data": "synthetic",
        "config": {"workload": wl.name, "batch": wl.B, "queries_per_seq": wl.S,
                   "end_pos": wl.end_pos, "compress_ratio": wl.ratio, "compressed_keys": wl.T,
                   "index_n_heads": wl.H, "index_head_dim": 128, "index_topk": wl.topk,
                   "candidate_topk_blocks": wl.ctb, "candidate_block_size": wl.cbs,
                   "publish": wl.publish, "key_cache_copies": n_caches,
                   "key_cache_layout": "paged" if args.paged else "contiguous",
                   "key_row": "fp8 e4m3, 132 bytes" if args.fp8 else "fp4 e2m1, 68 bytes",
                   "query_step": bool(args.q_step),
                   "prefill_publish": bool(args.prefill_publish)},
        "keys_scored_per_s": keys / step_s,
        "score_kernel_ms": score_ms,
        "score_kernel_ms_dist": percentiles(score_ms_all),
        "score_kernel_timed_steps": len(timed),
        "step_us_dist": percentiles(lat_us) if lat_us else None,
        "roofline": dict(roof, traffic=traffic, kernel=score_kernel_name(st),
                         algorithmic_bytes_per_launch=kb, algorithmic_flops_per_launch=kf,
                         scored_flops_per_launch=scored_flops(wl, st),
                         traffic_over_algorithmic=(traffic / kb if traffic and not prefill
                                                   else None),
                         step=step_roof),
    }
    if not args.no_cpu:
        line["cpu_baseline"] = cpu_baseline(wl, inp, args.cpu_seconds,
                                            threads=args.cpu_threads or None)
    else:
        line["cpu_baseline"] = None
    print(json.dumps(line), flush=True)
    del t_gen


if __name__ == "__main__":
    main()
