"""The seeded generator: shapes, determinism, and the sampled-rows path
drawing the same values as the full draw."""
import numpy as np

from sparse_attention_top_fp4_amd.inputs import Workload, generate, workload


def test_sampled_rows_equal_full_draw():
    wl = Workload(99, "t", B=5, S=1, H=8, T=300, start_pos=1199, ratio=4, topk=16)
    full = generate(wl)
    part = generate(wl, rows=[1, 4])
    assert np.array_equal(part["k"][0], full["k"][1])
    assert np.array_equal(part["k"][1], full["k"][4])
    assert np.array_equal(part["w"], full["w"]) and np.array_equal(part["q"], full["q"])


def test_workload_shapes():
    for cid, (R, T) in {0: (1, 512), 1: (64, 32768), 2: (32768, 8192), 3: (16, 65536),
                        4: (4, 262144)}.items():
        wl = workload(cid)
        assert (wl.R, wl.T) == (R, T)
    cl = workload(2).compress_lens()
    assert cl[0] == 0 and cl[3] == 1 and cl[-1] == 8192
    assert np.all(workload(1).compress_lens() == 32768)
