"""The benchmark's algorithmic accounting against closed forms, and its
one-GPU contract (CPU only).

Algorithmic bytes are what the method must move: the 68-byte key row of
every reachable (row, key) pair, each row's fp4 query heads (68 bytes a
head) and bf16 weights, and, for a whole step, the int32 indices it keeps
(plus level two, block ids and the key publish where the workload has
them).  The fp32 score scratch is an implementation cost and is excluded.

- batched decode at 128K: 64 rows x 32768 keys;
- causal prefill at 32K: compress_lens = (s + 1) // 4 over s < 32768, so
  each value c < 8192 occurs for four rows and 8192 for one; the launch
  that keeps no scores skips rows with compress_lens <= 2048 (closed form),
  but the algorithmic flops count every causal pair;
- two-level at 256K: 16 rows x 65536 keys at level one, 64 blocks of 128
  keys at level two;
- long decode at 1M with a publish: 4 rows x 262144 keys, wk 128 x 512.
"""
import os
import subprocess
import sys
from types import SimpleNamespace

import bench
from sparse_attention_top_fp4_amd.inputs import workload

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _causal_pairs(lo):
    """Sum of compress_lens over the prefill rows with compress_lens > lo."""
    return 4 * sum(range(lo + 1, 8192)) + 8192


def test_decode_bytes_closed_form():
    wl = workload(1)
    pairs = 64 * 32768
    kernel = pairs * 68 + 64 * 64 * 68 + 64 * 64 * 2
    assert bench.score_kernel_bytes(wl) == kernel == 142_893_056
    assert bench.step_bytes(wl) == kernel + 64 * 2048 * 4 == 143_417_344
    assert bench.score_kernel_flops(wl) == pairs * 64 * 128 * 2


def test_prefill_pairs_closed_form():
    wl = workload(2)
    kept = SimpleNamespace(fused=True, scores=object())
    lean = SimpleNamespace(fused=True, scores=None)
    assert int(bench.scored_compress_lens(wl, kept).sum()) == _causal_pairs(0) == 134_209_536
    assert int(bench.scored_compress_lens(wl, lean).sum()) == _causal_pairs(2048) == 125_816_832
    assert bench.scored_flops(wl, lean) == 125_816_832 * 64 * 256
    assert bench.score_kernel_flops(wl) == 134_209_536 * 64 * 256 == 2_198_889_037_824
    assert bench.step_flops(wl) == bench.score_kernel_flops(wl)


def test_two_level_and_publish_bytes_closed_form():
    wl = workload(3)
    l1 = 16 * 65536 * 68
    l2 = 16 * 64 * 128 * 68
    assert l1 == 71_303_168 and l2 == 8_912_896
    q, w = 16 * 64 * 68, 16 * 64 * 2
    assert bench.score_kernel_bytes(wl) == l1 + q + w
    assert bench.step_bytes(wl) == l1 + l2 + q + 2 * w + 16 * 64 * 4 + 2 * 16 * 2048 * 4
    wl = workload(4)
    keys = 4 * 262144 * 68
    assert bench.score_kernel_bytes(wl) == keys + 4 * 64 * 70
    assert bench.step_bytes(wl) == (keys + 4 * 64 * 70 + 4 * 2048 * 4
                                    + 128 * 512 * 2 + 4 * 512 * 2 + 4 * 68)


def test_timed_steps_are_spread():
    t = bench.timed_steps(20)
    assert len(t) == 8 and t[0] > 0 and t[-1] < 20 and t == sorted(set(t))
    t = bench.timed_steps(200)
    assert len(t) == 8 and t[0] > 0 and t[-1] < 200
    assert bench.timed_steps(3) == [0, 1, 2]


def _run_bench(args, env=None):
    e = dict(os.environ)
    e.update(env or {})
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], cwd=ROOT,
                          env=e, capture_output=True, text=True, timeout=120)


def test_more_than_one_gpu_is_refused():
    p = _run_bench(["--gpus", "2"])
    assert p.returncode == 2 and "one GPU" in p.stderr
    p = _run_bench([], env={"WORLD_SIZE": "4"})
    assert p.returncode == 2 and "one GPU" in p.stderr


def test_query_step_bytes_replace_the_quantised_heads():
    """With the query step, the step starts from bf16 heads (256 B a head)
    and raw weights (2 B) instead of quantised heads (68 B) and weights."""
    from sparse_attention_top_fp4_amd.inputs import workload
    wl = workload(1)
    assert bench.step_bytes(wl, q_step=True) - bench.step_bytes(wl) == wl.R * wl.H * (256 + 2 - 70)


def test_tsplit_needs_slices_that_divide_the_rows():
    """--tsplit checks its slicing before any GPU work (the long decode's
    262144 positions do not split in 3, and one slice is no split)."""
    for g in ("3", "1"):
        p = _run_bench(["--config", "4", "--tsplit", g, "--no-cpu"])
        assert p.returncode != 0 and "--tsplit" in p.stderr, (g, p.stderr[-300:])
