"""Synthetic serving trace for the periodic compression policy.

Concurrent sequences decode one token per step; every `period` steps a seeded
random subset of them is offered to the schedule (kara_schedule_step), and the
eligible ones are compressed in one batched kara_compress call on the GPU
("Technical Summary: Kara", Methodology 3, Periodic Compression Policy: the
trailing blocks of selected sequences are compressed every fixed number of
decoding steps).  The shapes follow the Distill-Llama-8B attention layout
(32 layers, 8 KV heads, 32 query heads, head dim 128).

Driver only: token appends, window queries and the random draws are synthetic
input generation; block allocation for appends uses the library's pool; every
compression step runs in libkara.

Inputs, all seeded: K ~ N(0,1)/sqrt(D) and V ~ N(0,1) per appended token;
planted high-similarity spans whose starts arrive with a mean gap of
`span_gap` tokens and whose lengths are U{span_len}; every span has one random
unit direction per (layer, KV head), added with amplitude
plant_scale * sqrt(D) * qk_std to the keys of its tokens and, when those
tokens are in a compressed window, to the window queries of that head's group
at the same positions.  Window queries are drawn when the window is
compressed (the pages do not say how query states are kept).
"""

from __future__ import annotations

import dataclasses
import math

import numpy as np
import torch

from . import kara


@dataclasses.dataclass
class TraceConfig:
    n_seqs: int = 128
    n_layers: int = 32
    n_q_heads: int = 32
    n_kv_heads: int = 8
    head_dim: int = 128
    block_size: int = 16
    window: int = 1024
    protect: int = 128
    top_k: int = 64
    retention: float = 0.2
    period: int = 128
    init_len: int = 2048
    max_len: int = 32768
    select_prob: float = 0.5
    span_gap: int = 256
    span_len: tuple = (4, 256)
    plant_scale: float = 3.0
    max_events: int = 0          # 0: run until the sequences reach max_len
    headroom_blocks: int = 64
    seed: int = 1004

    @property
    def budget(self):
        return int(math.floor(self.retention * (self.window - self.protect) + 1e-9))

    @property
    def qk_std(self):
        return self.head_dim ** -0.5


def simulate_schedule(cfg: TraceConfig):
    """Host-only replay of the selection and eligibility decisions, used to
    size the block pool before any GPU memory is touched: the library's own
    schedule (kara_schedule_step) and plan (kara_plan_lengths) on the lengths
    the trace will have.  Returns (n_events, peak blocks in use, largest
    per-event fresh-block demand)."""
    rng = np.random.default_rng(cfg.seed)
    S, bs, P = cfg.n_seqs, cfg.block_size, cfg.period
    params = kara.kara_params(cfg.window, cfg.protect, cfg.top_k, cfg.budget)
    phys = np.full(S, cfg.init_len, dtype=np.int64)
    wm = np.zeros(S, dtype=np.int64)
    logical = cfg.init_len
    n_events, peak, fresh_max, step = 0, 0, 0, 0
    while logical < cfg.max_len and (cfg.max_events == 0 or n_events < cfg.max_events):
        phys += P
        logical += P
        step += P
        n_events += 1
        peak = max(peak, int(sum(-(-L // bs) for L in phys)))
        sel = (rng.random(S) < cfg.select_prob).astype(np.uint8)
        batch = kara.kara_schedule_step(step, P, cfg.window, torch.from_numpy(phys.astype(np.int32)),
                                        torch.from_numpy(wm.astype(np.int32)), torch.from_numpy(sel))
        if not batch:
            continue
        new_lens, fresh = kara.kara_plan_lengths(params, bs, torch.tensor(phys[batch], dtype=torch.int32))
        fresh_max = max(fresh_max, int(fresh.sum()))
        phys[batch] = new_lens.numpy()
        wm[batch] = phys[batch] - cfg.protect
    return n_events, peak, fresh_max


class ServingTrace:
    """State of the trace on one GPU: pool, block tables, lengths, watermarks."""

    def __init__(self, cfg: TraceConfig, device="cuda"):
        self.cfg = cfg
        self.dev = torch.device(device)
        c = cfg
        self.G = c.n_q_heads // c.n_kv_heads
        n_events, peak, fresh_max = simulate_schedule(c)
        self.n_events = n_events
        self.NB = peak + fresh_max + c.headroom_blocks + c.n_seqs
        self.MB = -(-(c.max_len + c.period) // c.block_size)
        self.rng = np.random.default_rng(c.seed)                   # selection draws (same as the simulation)
        self.srng = np.random.default_rng(c.seed + 1)              # span metadata
        self.gen = torch.Generator(device=self.dev).manual_seed(c.seed + 2)
        self.pool = torch.empty((c.n_layers, 2, self.NB, c.n_kv_heads, c.block_size, c.head_dim),
                                dtype=torch.bfloat16, device=self.dev)
        self.blocks = kara.Pool(self.NB, torch.arange(self.NB, dtype=torch.int32))
        self.table = torch.full((c.n_seqs, self.MB), -1, dtype=torch.int32)
        self.phys = np.zeros(c.n_seqs, dtype=np.int64)
        self.watermark = np.zeros(c.n_seqs, dtype=np.int64)
        self.logical = 0
        # original positions of the physical tokens from each watermark on
        self.tail_orig = [[] for _ in range(c.n_seqs)]
        # planted spans per sequence: (start, length, id); directions per span
        self.spans = [[] for _ in range(c.n_seqs)]
        self.next_span_start = [int(self.srng.geometric(1.0 / c.span_gap)) for _ in range(c.n_seqs)]
        self.max_spans = int(c.max_len / c.span_gap * 2) + 16
        self.dirs = torch.zeros((c.n_seqs, self.max_spans, c.n_layers, c.n_kv_heads, c.head_dim),
                                dtype=torch.bfloat16, device=self.dev)
        self.amp = c.plant_scale * math.sqrt(c.head_dim) * c.qk_std
        self.events = 0
        self.step = 0
        self.append(c.init_len)

    # -- synthetic decoding ---------------------------------------------------

    def _span_ids(self, b, orig):
        """Planted-span id of each original position in `orig` (-1: none)."""
        if not self.spans[b]:
            return np.full(len(orig), -1, dtype=np.int64)
        starts = np.array([s0 for s0, _, _ in self.spans[b]], dtype=np.int64)
        ends = np.array([s0 + n for s0, n, _ in self.spans[b]], dtype=np.int64)
        orig = np.asarray(orig, dtype=np.int64)
        idx = np.searchsorted(starts, orig, side="right") - 1
        ok = (idx >= 0) & (orig < ends[np.maximum(idx, 0)])
        return np.where(ok, idx, -1)

    def _grow_spans(self, b, upto):
        c = self.cfg
        while self.next_span_start[b] < upto:
            k = len(self.spans[b])
            if k >= self.max_spans:
                break
            n = int(self.srng.integers(c.span_len[0], c.span_len[1] + 1))
            s0 = self.next_span_start[b]
            self.spans[b].append((s0, n, k))
            u = torch.randn((c.n_layers, c.n_kv_heads, c.head_dim), generator=self.gen, device=self.dev)
            self.dirs[b, k] = (u / u.norm(dim=-1, keepdim=True)).to(torch.bfloat16)
            self.next_span_start[b] = s0 + n + int(self.srng.geometric(1.0 / c.span_gap))

    def append(self, n_tokens):
        """Every sequence decodes n_tokens more tokens (K/V rows written into the pool)."""
        c = self.cfg
        bs = c.block_size
        blk_all, slot_all, sseq, sid, srow = [], [], [], [], []
        orig = np.arange(self.logical, self.logical + n_tokens, dtype=np.int64)
        for b in range(c.n_seqs):
            L = int(self.phys[b])
            need = -(-(L + n_tokens) // bs) - (-(-L // bs))
            if need:
                ids = self.blocks.alloc(need)
                e0 = -(-L // bs)
                self.table[b, e0:e0 + need] = torch.tensor(ids, dtype=torch.int32)
            self._grow_spans(b, self.logical + n_tokens)
            pos = L + np.arange(n_tokens, dtype=np.int64)
            trow = self.table[b].numpy()
            blk_all.append(trow[pos // bs].astype(np.int64))
            slot_all.append(pos % bs)
            ids = self._span_ids(b, orig)
            hit = np.nonzero(ids >= 0)[0]
            sseq.append(np.full(len(hit), b))
            sid.append(ids[hit])
            srow.append(b * n_tokens + hit)
            self.tail_orig[b].extend(orig.tolist())
            self.phys[b] = L + n_tokens
        self.logical += n_tokens
        blk = torch.from_numpy(np.concatenate(blk_all)).to(self.dev)
        slot = torch.from_numpy(np.concatenate(slot_all)).to(self.dev)
        N = blk.numel()
        srow = np.concatenate(srow)
        sdir = None
        if len(srow):
            sdir = self.dirs[torch.from_numpy(np.concatenate(sseq)).to(self.dev),
                             torch.from_numpy(np.concatenate(sid)).to(self.dev)].float() * self.amp
            srow = torch.from_numpy(srow).to(self.dev)
        for l in range(c.n_layers):
            k = torch.randn((N, c.n_kv_heads, c.head_dim), generator=self.gen, device=self.dev) * c.qk_std
            if sdir is not None:
                k[srow] += sdir[:, l]
            self.pool[l, 0, blk, :, slot, :] = k.to(torch.bfloat16)
            v = torch.randn((N, c.n_kv_heads, c.head_dim), generator=self.gen, device=self.dev)
            self.pool[l, 1, blk, :, slot, :] = v.to(torch.bfloat16)

    def window_queries(self, batch):
        """Window query states [nb, Lyr, W, Hq, D] for the sequences in `batch`."""
        c = self.cfg
        W, G = c.window, self.G
        q = torch.empty((len(batch), c.n_layers, W, c.n_q_heads, c.head_dim), dtype=torch.bfloat16,
                        device=self.dev)
        for i, b in enumerate(batch):
            qb = torch.randn((c.n_layers, W, c.n_q_heads, c.head_dim), generator=self.gen,
                             device=self.dev) * c.qk_std
            ids = self._span_ids(b, self.tail_orig[b][-W:])
            pos = np.nonzero(ids >= 0)[0]
            if len(pos):
                d = self.dirs[b, torch.from_numpy(ids[pos]).to(self.dev)].float() * self.amp  # [n, Lyr, Hkv, D]
                d = d.permute(1, 0, 2, 3).repeat_interleave(G, dim=2)                        # [Lyr, n, Hq, D]
                qb[:, torch.from_numpy(pos).to(self.dev)] += d
            q[i] = qb.to(torch.bfloat16)
        return q

    # -- compression events ---------------------------------------------------

    def next_event(self):
        """Advance `period` decode steps; returns the batch the schedule picks."""
        c = self.cfg
        self.append(c.period)
        self.step += c.period
        self.events += 1
        self.last_selected = (self.rng.random(c.n_seqs) < c.select_prob).astype(np.uint8)
        sel = torch.from_numpy(self.last_selected)
        lens = torch.from_numpy(self.phys.astype(np.int32))
        wm = torch.from_numpy(self.watermark.astype(np.int32))
        return kara.kara_schedule_step(self.step, c.period, c.window, lens, wm, sel)

    def batch_inputs(self, batch):
        """Host and device views of the batch's tables and lengths."""
        table_h = self.table[batch].contiguous()
        lens_h = torch.tensor([int(self.phys[b]) for b in batch], dtype=torch.int32)
        return table_h, table_h.to(self.dev), lens_h, lens_h.to(self.dev)

    def shape(self):
        c = self.cfg
        return kara.kara_shape(c.n_layers, c.n_q_heads, c.n_kv_heads, c.head_dim, c.block_size, kara.KARA_BF16)

    def params(self):
        c = self.cfg
        return kara.kara_params(c.window, c.protect, c.top_k, c.budget)

    def compress(self, batch, q_window, stream=None, outputs=None, stage_events=None):
        """One batched kara_compress call; updates tables, lengths, watermarks."""
        c = self.cfg
        table_h, table_d, lens_h, lens_d = self.batch_inputs(batch)
        new_table_h = torch.empty_like(table_h)
        new_table_d = torch.empty_like(table_d)
        new_lens_h = torch.empty_like(lens_h)
        shape, params = self.shape(), self.params()
        ws = torch.empty(max(kara.kara_workspace_bytes(shape, params, len(batch)), 256), dtype=torch.uint8,
                         device=self.dev)
        outputs = outputs or {}
        kara.kara_compress(shape, params, q_window, self.pool, table_h, table_d, lens_h, lens_d,
                           self.blocks, new_table_h, new_table_d, new_lens_h, ws, stream=stream,
                           scores_out=outputs.get("scores"), cand_out=outputs.get("cand"),
                           retained_out=outputs.get("retained"), stage_events=stage_events)
        for i, b in enumerate(batch):
            self.table[b] = new_table_h[i]
            L = int(lens_h[i])
            self.phys[b] = int(new_lens_h[i])
            self.watermark[b] = self.phys[b] - c.protect
            # protected tokens keep their original positions; earlier ones are compressed
            self.tail_orig[b] = self.tail_orig[b][-c.protect:] if c.protect else []
        return table_h, lens_h, new_table_h, new_lens_h

    def done(self):
        c = self.cfg
        return self.logical >= c.max_len or (c.max_events and self.events >= c.max_events)
