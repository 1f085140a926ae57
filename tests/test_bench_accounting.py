"""The benchmark's algorithmic accounting against closed forms, and its
one-GPU contract (CPU only).

- batched decode at 128K: 64 rows x 32768 keys, 68-byte key rows and 4-byte
  scores per pair plus each row's bf16 query (64 x 128) and weights (64);
- causal prefill at 32K: compress_lens = (s + 1) // 4 over s < 32768, so
  each value c < 8192 occurs for four rows and 8192 for one; the launch
  that keeps no scores skips rows with compress_lens <= 2048 (closed form).
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
    st = SimpleNamespace(fused=False, scores=object())
    pairs = 64 * 32768
    assert bench.score_kernel_bytes(wl, st) == pairs * (68 + 4) + 64 * (64 * 128 * 2 + 64 * 2)
    assert bench.score_kernel_bytes(wl, st) == 152_051_712
    assert bench.score_kernel_flops(wl, st) == pairs * 64 * 128 * 2


def test_prefill_pairs_closed_form():
    wl = workload(2)
    kept = SimpleNamespace(fused=True, scores=object())
    lean = SimpleNamespace(fused=True, scores=None)
    assert int(bench.scored_compress_lens(wl, kept).sum()) == _causal_pairs(0) == 134_209_536
    assert int(bench.scored_compress_lens(wl, lean).sum()) == _causal_pairs(2048) == 125_816_832
    assert bench.score_kernel_flops(wl, lean) == 125_816_832 * 64 * 256


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
