"""Helpers for the GPU parity tests: moving numpy arrays to and from the
device (bf16 as 16-bit patterns) and printing the case before each GPU step
so that a failing run names it."""
import sys

import numpy as np


def torch():
    import torch as _t
    return _t


def dev(a):
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch().from_numpy(a).cuda()


def host(t, dtype=None):
    a = t.detach().cpu().numpy()
    if dtype is not None:
        a = a.view(dtype)
    return a


def say(*args):
    print("[gpu-case]", *args, flush=True)
    sys.stdout.flush()


def sync():
    torch().cuda.synchronize()


def fp4_cache(k_bf16):
    """Quantise bf16 keys [B, T, 128] into a device cache [B, T, 68] with the
    library's quantiser (the HIP path's own cache)."""
    import sparse_attention_top_fp4_amd as idx
    t = torch()
    kd = dev(k_bf16)
    rows = t.empty(k_bf16.shape[:-1] + (68,), dtype=t.uint8, device="cuda")
    idx.idx_fp4_quant(kd, rows)
    return rows


def bits(x):
    return np.ascontiguousarray(x, np.float32).view(np.uint32)
