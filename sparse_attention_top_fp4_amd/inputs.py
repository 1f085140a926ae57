"""Seeded synthetic inputs shared by the tests, the benchmark and the oracle.

This module holds random draws, dtype conversion and the workload shapes
only -- none of the method's arithmetic (no quantisation, scoring, masking
or selection).  Both the HIP path and the CPU oracle consume the arrays it
returns; each quantises, scores and selects on its own.

The workloads follow the five configurations the indexer is exercised on
(tiny decode, batched decode at 128K tokens, causal prefill, two-level
selection, long-context decode with a key publish).  No dataset is involved:
every tensor is drawn from ``numpy.random.default_rng(seed)`` in a fixed
order (q, k, w, w2, latent, wk).
"""
from __future__ import annotations

import dataclasses

import numpy as np

HEAD_DIM = 128
ROW_BYTES = 68


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), round to nearest even."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(
        np.float32)


def normal_bf16(rng: np.random.Generator, shape, std: float = 1.0, chunk: int = 1 << 24):
    """N(0, std^2) draws rounded to bf16, generated in chunks to bound memory."""
    n = int(np.prod(shape))
    out = np.empty(n, np.uint16)
    for s in range(0, n, chunk):
        e = min(n, s + chunk)
        x = rng.standard_normal(e - s, dtype=np.float32)
        if std != 1.0:
            x *= np.float32(std)
        out[s:e] = bf16_bits(x)
    return out.reshape(shape)


def head_weights(rng, R, H, D=HEAD_DIM):
    """weights_proj output stand-in: N(0,1) bf16, times
    index_head_dim^-0.5 * index_n_heads^-0.5 in fp32, rounded to bf16 (the
    bf16 tensor-times-scalar of the Indexer's forward)."""
    n = bf16_to_f32(normal_bf16(rng, (R, H)))
    scale = np.float32(D ** -0.5 * H ** -0.5)
    return bf16_bits(n * scale)


@dataclasses.dataclass
class Workload:
    cid: int
    name: str
    B: int
    S: int
    H: int
    T: int            # compressed width end_pos // ratio
    start_pos: int
    ratio: int
    topk: int
    offset: int = 0
    ctb: int = 0      # candidate_topk_blocks (two-level only)
    cbs: int = 0      # candidate_block_size (two-level only)
    publish: bool = False
    din: int = 512
    rd: int = 64
    eps: float = 1e-6

    @property
    def R(self):
        return self.B * self.S

    @property
    def end_pos(self):
        return self.start_pos + self.S

    def compress_lens(self) -> np.ndarray:
        """Visible compressed positions per query row: (start_pos+s+1)//ratio."""
        s = np.arange(self.S, dtype=np.int64)
        cl = (self.start_pos + s + 1) // self.ratio
        return np.tile(cl, self.B).astype(np.int32)

    def seed(self):
        return 20260 + self.cid


# YaRN constants for the key-publish RoPE table: the pages name the
# parameters but print no values; these values are chosen here.
YARN = dict(theta=10000.0, factor=16.0, orig_len=65536, beta_fast=32.0, beta_slow=1.0)


def workload(cid: int) -> Workload:
    if cid == 0:
        return Workload(0, "tiny_decode", B=1, S=1, H=64, T=2048 // 4, start_pos=2047, ratio=4,
                        topk=256)
    if cid == 1:
        return Workload(1, "batched_decode_128k", B=64, S=1, H=64, T=131072 // 4,
                        start_pos=131071, ratio=4, topk=2048)
    if cid == 2:
        return Workload(2, "causal_prefill_32k", B=1, S=32768, H=64, T=32768 // 4, start_pos=0,
                        ratio=4, topk=2048)
    if cid == 3:
        return Workload(3, "two_level_256k", B=16, S=1, H=64, T=262144 // 4, start_pos=262143,
                        ratio=4, topk=2048, ctb=64, cbs=128)
    if cid == 4:
        return Workload(4, "long_decode_publish_1m", B=4, S=1, H=64, T=1048576 // 4,
                        start_pos=1048575, ratio=4, topk=2048, publish=True)
    raise ValueError(cid)


def generate(wl: Workload, seed=None, rows=None):
    """Draw the inputs of a workload.  Returns a dict of numpy arrays:
    q uint16 [R][H][128], k uint16 [B][T][128] (bf16 keys before the
    cache's fp4 round trip), w uint16 [R][H], cl int32 [R], and per
    workload w2 (two-level), latent uint16 [B][1][din], wk uint16
    [128][din], gamma float32 [128] (publish).  ``rows`` restricts k to the
    given sequences (for oracle samples of the large workloads); the draw
    order is unchanged, so the sampled values equal the full draw's."""
    rng = np.random.default_rng(wl.seed() if seed is None else seed)
    out = {}
    out["q"] = normal_bf16(rng, (wl.R, wl.H, HEAD_DIM))
    if rows is None:
        out["k"] = normal_bf16(rng, (wl.B, wl.T, HEAD_DIM))
    else:
        per = wl.T * HEAD_DIM
        ks = []
        for b in range(wl.B):
            if b in rows:
                ks.append(normal_bf16(rng, (wl.T, HEAD_DIM)))
            else:
                rng.standard_normal(per, dtype=np.float32)  # keep the stream aligned
        out["k"] = np.stack(ks) if ks else np.empty((0, wl.T, HEAD_DIM), np.uint16)
    out["w"] = head_weights(rng, wl.R, wl.H)
    if wl.ctb:
        out["w2"] = head_weights(rng, wl.R, wl.H)
    if wl.publish:
        out["latent"] = normal_bf16(rng, (wl.B, 1, wl.din))
        out["wk"] = normal_bf16(rng, (HEAD_DIM, wl.din), std=0.02)
        out["gamma"] = np.ones(HEAD_DIM, np.float32)
    out["cl"] = wl.compress_lens()
    return out


def publish_inputs(wl: Workload, groups: int, seed: int):
    """Key-publish inputs for `groups` groups per sequence, from their own
    seeded stream: latent uint16 [B][groups][din] N(0,1) bf16, wk uint16
    [128][din] N(0, 0.02^2) bf16, gamma float32 [128] ones."""
    rng = np.random.default_rng(seed)
    return {"latent": normal_bf16(rng, (wl.B, groups, wl.din)),
            "wk": normal_bf16(rng, (HEAD_DIM, wl.din), std=0.02),
            "gamma": np.ones(HEAD_DIM, np.float32)}


def small_case(seed, B, S, H, T, start_pos=None, ratio=4, tcap=None):
    """A fuzz-sized decode/prefill case: q, k (bf16), w, and compress_lens
    for rows r = b*S + s.  start_pos None gives decode at end_pos = T*ratio
    (S must be 1) or, with S > 1, a prefill from 0."""
    rng = np.random.default_rng(seed)
    tcap = T if tcap is None else tcap
    q = normal_bf16(rng, (B * S, H, HEAD_DIM))
    k = normal_bf16(rng, (B, tcap, HEAD_DIM))
    w = head_weights(rng, B * S, H)
    if start_pos is None:
        start_pos = T * ratio - 1 if S == 1 else 0
    s = np.arange(S)
    cl = np.tile((start_pos + s + 1) // ratio, B).astype(np.int32)
    return dict(q=q, k=k, w=w, cl=cl, start_pos=start_pos)


def yarn_params():
    return dict(YARN)


def cache_bytes(B, T):
    return B * T * ROW_BYTES


__all__ = ["bf16_bits", "bf16_to_f32", "normal_bf16", "head_weights", "Workload", "workload",
           "generate", "small_case", "YARN", "yarn_params"]
