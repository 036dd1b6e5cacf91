"""Seeded synthetic workloads shaped like the models and settings the Kara pages
evaluate (Qwen3-4B, Qwen3-14B and Distill-Llama-8B attention shapes; long
reasoning traces served from a paged KV cache).

This module only draws inputs: window query states, a paged K/V pool with a
fragmented block table, sequence lengths, a free list and, where a workload
asks for it, planted high-similarity spans.  It holds none of the compression
arithmetic, so both the HIP path and the CPU checker can take their inputs
from here.

Layouts (shared by every consumer):
  q_window  [S, Lyr, W, Hq, D]            bf16 (fp32 for the tiny workload)
  pool      [Lyr, 2, NB, Hkv, bs, D]      K = index 0, V = index 1
  table     [S, MB] int32 block ids; entries past a sequence's last block are -1
  lens      [S] int32
  free_ids  list of the pool's free block ids, front first

Entries of the table that precede the window's first (boundary) block are never
read by the compression step.  With ``materialize_prefix=False`` they hold -2
and no pool memory backs them, which keeps the 128-sequence Qwen3-14B-shaped
workload inside one GPU's memory.
"""

from __future__ import annotations

import dataclasses
import math
from typing import Optional

import torch


@dataclasses.dataclass
class Workload:
    name: str
    n_seqs: int
    n_layers: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    block_size: int
    window: int
    protect: int
    top_k: int
    budget: int
    dtype: torch.dtype
    q_window: torch.Tensor
    pool: torch.Tensor
    table: torch.Tensor          # int32, on the same device as pool
    lens: torch.Tensor           # int32, on the same device as pool
    free_ids: list
    spans: list                  # per sequence: list of (start, length) in window-local positions
    seed: int

    @property
    def n_blocks(self):
        return self.pool.shape[2]

    @property
    def max_blocks(self):
        return self.table.shape[1]

    @property
    def region(self):
        return self.window - self.protect

    @property
    def n_units(self):
        return self.n_seqs * self.n_layers * self.n_kv_heads

    def to(self, device):
        d = dataclasses.replace(self)
        d.q_window = self.q_window.to(device)
        d.pool = self.pool.to(device)
        d.table = self.table.to(device)
        d.lens = self.lens.to(device)
        return d


# Workload definitions: (S, Lyr, Hq, Hkv, D, bs, W, B, K, retention, len range, dtype, planted)
CONFIGS = {
    0: dict(name="tiny-fp32", n_seqs=1, n_layers=1, n_q_heads=4, n_kv_heads=2, head_dim=64,
            block_size=16, window=64, protect=8, top_k=8, budget=16, lens=(256, 256),
            dtype=torch.float32, qk_std=1.0, planted=0, pool_blocks=32),
    1: dict(name="qwen3-4b-1layer", n_seqs=1, n_layers=1, n_q_heads=32, n_kv_heads=8, head_dim=128,
            block_size=16, window=1024, protect=128, top_k=64, retention=0.2, lens=(8192, 8192),
            dtype=torch.bfloat16, qk_std=128 ** -0.5, planted=4),
    2: dict(name="qwen3-4b-36layer-b32", n_seqs=32, n_layers=36, n_q_heads=32, n_kv_heads=8,
            head_dim=128, block_size=16, window=1024, protect=128, top_k=64, retention=0.2,
            lens=(4096, 16384), dtype=torch.bfloat16, qk_std=128 ** -0.5, planted=4),
    # one compression event of the Distill-Llama-8B-shaped serving trace, as a
    # static batch (the trace itself lives in trace.py)
    4: dict(name="distill-llama-8b-event-b16", n_seqs=16, n_layers=32, n_q_heads=32, n_kv_heads=8,
            head_dim=128, block_size=16, window=1024, protect=128, top_k=64, retention=0.2,
            lens=(2048, 13400), dtype=torch.bfloat16, qk_std=128 ** -0.5, planted=4, span_len=(4, 256)),
    3: dict(name="qwen3-14b-40layer-b128", n_seqs=128, n_layers=40, n_q_heads=40, n_kv_heads=8,
            head_dim=128, block_size=16, window=2048, protect=256, top_k=128, retention=0.3,
            lens=(8192, 32768), dtype=torch.bfloat16, qk_std=128 ** -0.5, planted=0,
            materialize_prefix=False),
}


def budget_for(window, protect, retention):
    """Kept tokens of the compressible region for a retention ratio (rounded down)."""
    return int(math.floor(retention * (window - protect) + 1e-9))


def _plant_spans(gen, n_spans, region, lo=8, hi=64):
    """Non-overlapping spans of length U{lo..hi} at uniform positions in [0, region)."""
    spans = []
    tries = 0
    while len(spans) < n_spans and tries < 10000:
        tries += 1
        n = int(torch.randint(lo, hi + 1, (1,), generator=gen))
        s = int(torch.randint(0, region - n + 1, (1,), generator=gen))
        if all(s + n <= a or a + m <= s for a, m in spans):
            spans.append((s, n))
    return sorted(spans)


def make_workload(cfg=None, seed=None, device="cpu", **over) -> Workload:
    """Build a workload from a numbered config, with keyword overrides.

    Recognised keys: name, n_seqs, n_layers, n_q_heads, n_kv_heads, head_dim,
    block_size, window, protect, top_k, budget or retention, lens=(lo, hi) or
    an explicit list, dtype, qk_std, v_std, planted (spans per sequence),
    span_len=(lo, hi), plant_scale (multiple of qk_std*sqrt(D)), headroom
    (extra free blocks as a fraction), pool_blocks, materialize_prefix.
    """
    p = dict(CONFIGS[cfg]) if cfg is not None else {}
    p.update(over)
    seed = (1000 + (cfg or 0)) if seed is None else seed
    S, Lyr = p["n_seqs"], p["n_layers"]
    Hq, Hkv, D, bs = p["n_q_heads"], p["n_kv_heads"], p["head_dim"], p["block_size"]
    W, B = p["window"], p["protect"]
    C = W - B
    R = p["budget"] if "budget" in p else budget_for(W, B, p["retention"])
    K = p["top_k"]
    dtype = p.get("dtype", torch.bfloat16)
    qk_std = p.get("qk_std", D ** -0.5)
    v_std = p.get("v_std", 1.0)
    materialize = p.get("materialize_prefix", True)
    dev = torch.device(device)

    gcpu = torch.Generator().manual_seed(seed)
    lens_spec = p["lens"]
    if isinstance(lens_spec, tuple):
        lo, hi = lens_spec
        lens = [int(x) for x in torch.randint(lo, hi + 1, (S,), generator=gcpu)]
    else:
        lens = [int(x) for x in lens_spec]
    if any(L < W for L in lens):
        raise ValueError("every sequence needs at least W tokens")

    # Block accounting: materialised blocks per sequence, plus fresh-block headroom.
    first_blk = [((L - W) // bs) if not materialize else 0 for L in lens]
    n_blk = [math.ceil(L / bs) for L in lens]
    used = sum(n - f for n, f in zip(n_blk, first_blk))
    fresh = sum(math.ceil(((L - W) % bs + R + B) / bs) for L in lens)
    NB = p.get("pool_blocks") or int(math.ceil((used + fresh) * (1.0 + p.get("headroom", 0.1)))) + 1
    if NB < used + fresh:
        raise ValueError("pool too small for the workload")
    perm = torch.randperm(NB, generator=gcpu).tolist()
    MB = max(n_blk)
    table = torch.full((S, MB), -1, dtype=torch.int32)
    cur = 0
    for b in range(S):
        if first_blk[b] > 0:
            table[b, :first_blk[b]] = -2
        m = n_blk[b] - first_blk[b]
        table[b, first_blk[b]:n_blk[b]] = torch.tensor(perm[cur:cur + m], dtype=torch.int32)
        cur += m
    free_ids = perm[cur:]

    # Dense states.  Drawn in float32 on the target device, stored in `dtype`.
    gdev = torch.Generator(device=dev).manual_seed(seed + 1)
    q_window = torch.empty((S, Lyr, W, Hq, D), dtype=dtype, device=dev)
    for b in range(S):
        for l in range(Lyr):
            q_window[b, l] = (torch.randn((W, Hq, D), generator=gdev, device=dev) * qk_std).to(dtype)
    pool = torch.empty((Lyr, 2, NB, Hkv, bs, D), dtype=dtype, device=dev)
    for l in range(Lyr):
        for kv, std in ((0, qk_std), (1, v_std)):
            pool[l, kv] = (torch.randn((NB, Hkv, bs, D), generator=gdev, device=dev) * std).to(dtype)

    # Planted spans: per sequence, shared by all layers and heads; per (layer,
    # KV head, span) one random unit direction added to the keys of the span
    # and to the queries of that head's group at the same positions.
    spans = [[] for _ in range(S)]
    n_plant = p.get("planted", 0)
    if n_plant:
        slo, shi = p.get("span_len", (8, 64))
        amp = p.get("plant_scale", 3.0) * qk_std * math.sqrt(D)
        G = Hq // Hkv
        for b in range(S):
            spans[b] = _plant_spans(gcpu, n_plant, C, slo, shi)
            start = lens[b] - W
            toks = torch.tensor([start + t for s0, n in spans[b] for t in range(s0, s0 + n)], dtype=torch.long)
            locs = torch.tensor([t for s0, n in spans[b] for t in range(s0, s0 + n)], dtype=torch.long)
            sid = torch.tensor([k for k, (s0, n) in enumerate(spans[b]) for _ in range(n)], dtype=torch.long)
            blk = table[b].long()[toks // bs].to(dev)
            off = (toks % bs).to(dev)
            for l in range(Lyr):
                u = torch.randn((len(spans[b]), Hkv, D), generator=gcpu)
                u = (u / u.norm(dim=-1, keepdim=True) * amp).to(dev)
                add = u[sid.to(dev)]                                        # [n_tok, Hkv, D]
                kb = pool[l, 0, blk, :, off, :].float()                     # [n_tok, Hkv, D]
                pool[l, 0, blk, :, off, :] = (kb + add).to(dtype)
                qa = add.repeat_interleave(G, dim=1)                         # [n_tok, Hq, D]
                qb = q_window[b, l, locs.to(dev)].float()
                q_window[b, l, locs.to(dev)] = (qb + qa).to(dtype)

    return Workload(
        name=p.get("name", "custom"), n_seqs=S, n_layers=Lyr, n_q_heads=Hq, n_kv_heads=Hkv,
        head_dim=D, block_size=bs, window=W, protect=B, top_k=K, budget=R, dtype=dtype,
        q_window=q_window, pool=pool, table=table.to(dev), lens=torch.tensor(lens, dtype=torch.int32, device=dev),
        free_ids=free_ids, spans=spans, seed=seed)


def random_scores(n_units, region, seed, kind="normal", device="cpu"):
    """Float32 score rows for exercising the selection stages on their own.

    kind: "normal" (distinct values), "ties" (three distinct values, many
    ties), "coarse" (values on a grid of 1/64, frequent ties), "flat" (one
    value everywhere), "spiky" (mostly tiny values with a few large ones).
    """
    g = torch.Generator().manual_seed(seed)
    if kind == "normal":
        s = torch.rand((n_units, region), generator=g) * 4.0
    elif kind == "ties":
        s = torch.randint(0, 3, (n_units, region), generator=g).float() * 0.5 + 1.0
    elif kind == "coarse":
        s = torch.randint(0, 256, (n_units, region), generator=g).float() / 64.0
    elif kind == "flat":
        s = torch.full((n_units, region), 4.0)
    elif kind == "spiky":
        s = torch.rand((n_units, region), generator=g) * 1e-3
        hot = torch.rand((n_units, region), generator=g) < 0.05
        s = torch.where(hot, s * 4000.0 + 1.0, s)
    else:
        raise ValueError(kind)
    return s.to(torch.float32).to(device)


def random_retained(n_units, region, budget, seed):
    """Ascending random position sets of size ``budget`` per unit, int32."""
    g = torch.Generator().manual_seed(seed)
    out = torch.empty((n_units, budget), dtype=torch.int32)
    for u in range(n_units):
        out[u] = torch.sort(torch.randperm(region, generator=g)[:budget]).values.to(torch.int32)
    return out
