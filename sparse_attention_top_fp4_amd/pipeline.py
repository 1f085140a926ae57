"""One step of the Indexer hot path on device buffers, composed from the C
ABI calls (argument marshalling and buffer bookkeeping only).

A step follows the Indexer's forward ("DeepSeek V4.1" page, class Indexer):
  [key publish]  -> score -> [candidate block select -> level-one top-k ->
  level-two score inside the candidate blocks] -> top-k
For the two-level workload the level-one layer (the candidate source) keeps
its own top-k as the Indexer does, and the level-two layer scores with its
own weights inside the selected blocks.
"""
from __future__ import annotations

import ctypes

import numpy as np

from . import (PAGE_ROWS, current_stream_handle, idx_clear_key_hist, idx_fp4_quant,
               idx_publish_score_paged, idx_publish_score_fp8,
               idx_fp8_quant, idx_publish_keys, idx_publish_keys_fp8, idx_publish_keys_paged,
               idx_publish_score, idx_score_select_blocks, idx_score_topk_candidates,
               idx_score_fp8, idx_q_rope_quant, idx_score, idx_score_paged,
               idx_score_q4, idx_score_topk, idx_score_topk_q4, idx_score_qrope,
               idx_score_topk_qrope,
               idx_score_topk_paged, idx_select_candidate_blocks, idx_select_workspace_size,
               idx_topk, idx_topk_candidates, idx_two_level_topk,
               idx_timing_arm, idx_topk_workspace_size, idx_yarn_cos_sin)
from .inputs import YARN


def _torch():
    import torch
    return torch


def to_device(a: np.ndarray):
    torch = _torch()
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).cuda()


def quantize_cache(k_bf16_dev, fp8=False):
    """bf16 keys [B, T, 128] on device -> 68-byte fp4 rows [B, T, 68], or
    132-byte FP8 rows [B, T, 132]."""
    torch = _torch()
    rb = 132 if fp8 else 68
    rows = torch.empty(tuple(k_bf16_dev.shape[:-1]) + (rb,), dtype=torch.uint8,
                       device=k_bf16_dev.device)
    (idx_fp8_quant if fp8 else idx_fp4_quant)(k_bf16_dev, rows)
    return rows


class IndexerStep:
    """Device state of one workload: inputs, the fp4 key cache(s), outputs and
    workspaces.  ``n_caches`` > 1 keeps several copies of the key cache and
    cycles through them step by step (benchmarks use it so that consecutive
    steps do not read keys left in the 256 MB last-level cache)."""

    # rows up to this width are scored and ranked in one launch
    FUSED_MAX_T = 8192

    def __init__(self, wl, inp: dict, n_caches: int = 1, keep_scores: bool = True,
                 paged: bool = False, q_step: bool = False, publish=None, fp8: bool = False):
        torch = _torch()
        self.wl = wl
        R, T = wl.R, wl.T
        # fp8: the key cache holds FP8 rows (132 bytes) and every step scores
        # them with idx_score_fp8 (no fused launch, no pages, no query step)
        self.fp8 = fp8
        if fp8 and (paged or q_step):
            raise ValueError("the FP8 cache is contiguous and takes bf16 query heads")
        self.q = to_device(inp["q"])
        self.w = to_device(inp["w"])
        self.cl = to_device(inp["cl"])
        k = to_device(inp["k"])
        self.caches = [quantize_cache(k, fp8=fp8)]
        del k
        for _ in range(1, n_caches):
            self.caches.append(self.caches[0].clone())
        self.cur = 0
        # paged: each cache copy becomes a pool of pages of PAGE_ROWS rows,
        # the sequences' logical pages in a seeded random order
        self.paged = paged
        if paged:
            npg = (T + PAGE_ROWS - 1) // PAGE_ROWS
            perm = np.random.default_rng(7).permutation(wl.B * npg).astype(np.int32)
            self.block_table = to_device(perm.reshape(wl.B, npg))
            dst = torch.from_numpy(perm.astype(np.int64)).cuda()
            pools = []
            for kc in self.caches:
                padded = torch.zeros((wl.B, npg * PAGE_ROWS, 68), dtype=torch.uint8, device="cuda")
                padded[:, :kc.shape[1]] = kc
                pool = torch.empty((wl.B * npg, PAGE_ROWS * 68), dtype=torch.uint8, device="cuda")
                pool[dst] = padded.reshape(wl.B * npg, PAGE_ROWS * 68)
                pools.append(pool)
            self.caches = pools
        # single-level rows up to FUSED_MAX_T take the fused score + top-k
        # launch; its scores are written only when kept
        self.fused = not wl.ctb and T <= self.FUSED_MAX_T and not fp8
        self.scores = None
        if keep_scores or not self.fused:
            self.scores = torch.empty((R, T), dtype=torch.float32, device="cuda")
        self.kout = min(wl.topk, T)
        self.out = torch.empty((R, self.kout), dtype=torch.int32, device="cuda")
        self.topk_ws = self._ws(idx_topk_workspace_size(R, T, wl.topk))
        # first-digit histogram of the scores, filled by the score kernel and
        # reset by the top-k that consumes it; cleared once here
        self.key_hist = None
        if not self.fused:
            self.key_hist = torch.empty((R, 2048), dtype=torch.int32, device="cuda")
            idx_clear_key_hist(self.key_hist)
        self.two_level = bool(wl.ctb)
        if self.two_level:
            self.w2 = to_device(inp["w2"])
            nb = (T + wl.cbs - 1) // wl.cbs
            self.ids = torch.empty((R, min(wl.ctb, nb)), dtype=torch.int32, device="cuda")
            self.sel_ws = self._ws(idx_select_workspace_size(R, T, wl.ctb, wl.cbs))
            self.scores2 = torch.empty((R, T), dtype=torch.float32, device="cuda")
            self.out_l1 = torch.empty((R, self.kout), dtype=torch.int32, device="cuda")
        # q_step: the step starts from the query heads before RoPE (the
        # workload's q taken as such) and runs the query step first; the
        # workload's weights are already scaled, so the weight scale is 1
        self.q_step = q_step
        # the query step runs inside the score launch on one-level
        # contiguous fp4 steps (idx_score_qrope, idx_score_topk_qrope); the
        # others run it as its own launch into these buffers
        self.qrope = q_step and not paged and not self.two_level and not fp8
        if q_step:
            H = wl.H
            self.q_rows = torch.empty((R, H, 68), dtype=torch.uint8, device="cuda")
            self.q_rt = torch.empty((R, H, 128), dtype=torch.int16, device="cuda")
            self.w_q = torch.empty((R, H), dtype=torch.int16, device="cuda")
            P = wl.start_pos + wl.S
            self.cos_sin_q = to_device(idx_yarn_cos_sin(P, wl.rd, YARN["theta"], YARN["factor"],
                                                        YARN["orig_len"], YARN["beta_fast"],
                                                        YARN["beta_slow"]))
        # publish: None follows the workload; True on a prefill workload
        # publishes its S / ratio groups (inp must hold their latent)
        self.publish = bool(wl.publish) if publish is None else bool(publish)
        if self.publish:
            self.latent = to_device(inp["latent"])
            self.wk = to_device(inp["wk"])
            self.gamma = to_device(inp["gamma"])
            groups = 1 if wl.start_pos > 0 else wl.S // wl.ratio
            pos_max = (wl.start_pos + 1 - wl.ratio if wl.start_pos > 0
                       else (groups - 1) * wl.ratio)
            P = pos_max + 1
            self.cos_sin = to_device(idx_yarn_cos_sin(P, wl.rd, YARN["theta"], YARN["factor"],
                                                      YARN["orig_len"], YARN["beta_fast"],
                                                      YARN["beta_slow"]))

        # the decode publish of the last scored key joins the score launch
        # (idx_publish_score, idx_publish_score_paged, idx_publish_score_fp8)
        # with bf16 queries
        self.publish_in_score = (self.publish and wl.S == 1 and wl.start_pos > 0 and
                                 wl.start_pos // wl.ratio == T - 1 and
                                 not self.fused and not (q_step and not wl.ctb) and
                                 wl.din <= 2048)

        # level two keeps its scores per candidate slot (scores2[r][v]) on
        # contiguous fp4 caches with bf16 queries
        self.l2_compact = (self.two_level and not paged and not fp8 and
                           not (q_step and not wl.ctb))
        # ... and then runs after the level-one select as one call
        # (idx_two_level_topk), whose two rankings may run side by side: level
        # two counts into a histogram of its own
        self.key_hist2 = None
        if self.l2_compact:
            self.key_hist2 = torch.empty((R, 2048), dtype=torch.int32, device="cuda")
            idx_clear_key_hist(self.key_hist2)

        # every step's calls, marshalled once per key-cache copy
        self._plans = [self._plan(kc) for kc in self.caches]

    @staticmethod
    def _ws(nbytes):
        torch = _torch()
        return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device="cuda")

    @property
    def k_cache(self):
        return self.caches[self.cur]

    def step(self, stream=None, time_slot=None):
        """Issue one step on `stream` (default: torch's current stream),
        asynchronously.  time_slot: when given, the (level-one) score launch
        records its kernel's start and end into that library event pair
        (idx_timing_read reads it).  The step's calls were marshalled once
        per key-cache copy (BoundCall), so a step costs the host little more
        than the launches themselves."""
        plan, score_at = self._plans[self.cur]
        h = current_stream_handle() if stream is None else ctypes.c_void_p(stream.cuda_stream)
        for i, call in enumerate(plan):
            if i == score_at and time_slot is not None:
                idx_timing_arm(time_slot)
            call(h)
        self.cur = (self.cur + 1) % len(self.caches)

    def _plan(self, kc):
        """The calls of one step on key cache `kc`, bound (not issued), and
        the position of the (level-one) score launch among them."""
        wl = self.wl
        calls = []
        b = dict(bind=True)
        # a decode step whose new key is the last scored position publishes
        # it inside the score launch (one extra workgroup per sequence)
        pub_in_score = self.publish_in_score
        if self.publish and not pub_in_score:
            if self.paged:
                calls.append(idx_publish_keys_paged(self.latent, self.wk, self.gamma, self.cos_sin,
                                                    wl.start_pos, wl.ratio, wl.eps, kc,
                                                    self.block_table, wl.T, rd=wl.rd, **b))
            else:
                pub = idx_publish_keys_fp8 if self.fp8 else idx_publish_keys
                calls.append(pub(self.latent, self.wk, self.gamma, self.cos_sin, wl.start_pos,
                                 wl.ratio, wl.eps, kc, rd=wl.rd, **b))
        q, w = self.q, self.w
        q4 = None  # the quantised heads, when the score takes them directly
        if self.qrope:
            qs = dict(w_scale=1.0, cos_sin=self.cos_sin_q, start_pos=wl.start_pos, rd=wl.rd)
            score_at = len(calls)
            if self.fused:
                calls.append(idx_score_topk_qrope(q, w, qs["w_scale"], qs["cos_sin"],
                                                  qs["start_pos"], kc, wl.B, wl.S, wl.T, self.cl,
                                                  wl.topk, wl.offset, self.out,
                                                  scores=self.scores, rd=qs["rd"], **b))
                return calls, score_at
            calls.append(idx_score_qrope(q, w, qs["w_scale"], qs["cos_sin"], qs["start_pos"], kc,
                                         wl.B, wl.S, wl.T, self.cl, self.scores,
                                         key_hist=self.key_hist, rd=qs["rd"], **b))
            calls.append(idx_topk(self.scores, wl.T, self.cl, wl.topk, wl.offset, self.out,
                                  workspace=self.topk_ws, key_hist=self.key_hist, **b))
            return calls, score_at
        if self.q_step:
            # the score takes the rows directly; the paged and level-two
            # scores take the bf16 round trip
            direct = not self.paged and not self.two_level
            calls.append(idx_q_rope_quant(self.q, self.w, 1.0, self.cos_sin_q, wl.start_pos,
                                          wl.S, self.q_rows, self.w_q,
                                          q_roundtrip=None if direct else self.q_rt, rd=wl.rd,
                                          **b))
            w = self.w_q
            if direct:
                q4 = self.q_rows
            else:
                q = self.q_rt
        score_at = len(calls)
        selected = False  # the candidate blocks chosen with the level-one score
        if self.fused:
            if self.paged:
                calls.append(idx_score_topk_paged(q, w, kc, self.block_table, wl.B, wl.S, wl.T,
                                                  self.cl, wl.topk, wl.offset, self.out,
                                                  scores=self.scores, **b))
            elif q4 is not None:
                calls.append(idx_score_topk_q4(q4, w, kc, wl.B, wl.S, wl.T, self.cl, wl.topk,
                                               wl.offset, self.out, scores=self.scores, **b))
            else:
                calls.append(idx_score_topk(q, w, kc, wl.B, wl.S, wl.T, self.cl, wl.topk,
                                            wl.offset, self.out, scores=self.scores, **b))
            return calls, score_at
        if self.paged and pub_in_score:
            calls.append(idx_publish_score_paged(self.latent, self.wk, self.gamma, self.cos_sin,
                                                 wl.start_pos, wl.ratio, wl.eps, q, w, kc,
                                                 self.block_table, wl.T, self.cl, self.scores,
                                                 key_hist=self.key_hist, rd=wl.rd, **b))
        elif self.paged:
            calls.append(idx_score_paged(q, w, kc, self.block_table, wl.B, wl.S, wl.T, self.cl,
                                         self.scores, key_hist=self.key_hist, **b))
        elif q4 is not None:
            calls.append(idx_score_q4(q4, w, kc, wl.B, wl.S, wl.T, self.cl, self.scores,
                                      key_hist=self.key_hist, **b))
        elif pub_in_score:
            pub_score = idx_publish_score_fp8 if self.fp8 else idx_publish_score
            calls.append(pub_score(self.latent, self.wk, self.gamma, self.cos_sin,
                                   wl.start_pos, wl.ratio, wl.eps, q, w, kc, wl.T, self.cl,
                                   self.scores, key_hist=self.key_hist, rd=wl.rd, **b))
        elif self.two_level and not self.fp8:
            # level one: the score launch also writes the block maxima and
            # one wave per row selects the candidate blocks
            selected = True
            calls.append(idx_score_select_blocks(q, w, kc, wl.B, wl.S, wl.T, self.cl, self.scores,
                                                 wl.ctb, wl.cbs, self.ids, self.sel_ws,
                                                 key_hist=self.key_hist, **b))
        else:
            score = idx_score_fp8 if self.fp8 else idx_score
            calls.append(score(q, w, kc, wl.B, wl.S, wl.T, self.cl, self.scores,
                               key_hist=self.key_hist, **b))
        if self.two_level:
            if not selected:
                calls.append(idx_select_candidate_blocks(self.scores, wl.T, self.cl, wl.ctb,
                                                         wl.cbs, self.ids, workspace=self.sel_ws,
                                                         **b))
            if self.l2_compact:
                # the level-one top-k, and level two's slot scores (no -inf
                # fill of the rows) and top-k, in one call
                calls.append(idx_two_level_topk(self.scores, self.key_hist, self.out_l1,
                                                self.topk_ws, q, self.w2, kc, wl.B, wl.S, wl.T,
                                                self.cl, self.ids, wl.cbs, self.scores2,
                                                self.key_hist2, wl.topk, wl.offset, self.out,
                                                **b))
                return calls, score_at
            calls.append(idx_topk(self.scores, wl.T, self.cl, wl.topk, wl.offset, self.out_l1,
                                  workspace=self.topk_ws, key_hist=self.key_hist, **b))
            # level two: only the candidate positions hold finite scores; the
            # histogram, reset by the level-one top-k, now counts them
            if self.paged:
                calls.append(idx_score_paged(q, self.w2, kc, self.block_table, wl.B, wl.S, wl.T,
                                             self.cl, self.scores2, cand_blocks=self.ids,
                                             cand_block_size=wl.cbs, key_hist=self.key_hist,
                                             **b))
            else:
                score = idx_score_fp8 if self.fp8 else idx_score
                calls.append(score(q, self.w2, kc, wl.B, wl.S, wl.T, self.cl, self.scores2,
                                   cand_blocks=self.ids, cand_block_size=wl.cbs,
                                   key_hist=self.key_hist, **b))
            calls.append(idx_topk_candidates(self.scores2, wl.T, self.cl, self.ids, wl.cbs,
                                             wl.topk, wl.offset, self.out,
                                             key_hist=self.key_hist, **b))
        else:
            calls.append(idx_topk(self.scores, wl.T, self.cl, wl.topk, wl.offset, self.out,
                                  workspace=self.topk_ws, key_hist=self.key_hist, **b))
        return calls, score_at

    def level_two_rows(self):
        """The level-two scores as full rows [R, T]: scores2 itself, or, when
        level two keeps them per candidate slot, scattered to their
        positions (-inf at every other position and at or past
        compress_lens, as the full-row form leaves them)."""
        if not self.l2_compact:
            return self.scores2
        torch = _torch()
        wl = self.wl
        R, T, cbs = wl.R, wl.T, wl.cbs
        V = self.ids.shape[1] * cbs
        v = torch.arange(V, device="cuda")
        blk = self.ids.long()[:, v // cbs]
        pos = blk * cbs + (v % cbs)[None, :]
        ok = (blk >= 0) & (pos < T) & (pos < self.cl.long()[:, None].clamp(0, T))
        full = torch.full((R, T + 1), float("-inf"), dtype=torch.float32, device="cuda")
        idx = torch.where(ok, pos, torch.full_like(pos, T))  # invalid slots land in column T
        full.scatter_(1, idx, torch.where(ok, self.scores2[:, :V], full[:, :1].expand(-1, V)))
        return full[:, :T].contiguous()

    def keys_scored(self):
        """Algorithmic (query, key) pairs scored per step.  The fused launch
        without scores kept does not score rows whose compress_lens is at
        most k_out (their result is the closed form)."""
        wl = self.wl
        cl = np.minimum(wl.compress_lens().astype(np.int64), wl.T)
        if self.fused and self.scores is None:
            cl = np.where(cl > self.kout, cl, 0)
        n = int(cl.sum())
        if self.two_level:
            n += wl.R * min(wl.ctb * wl.cbs, wl.T)
        return n
