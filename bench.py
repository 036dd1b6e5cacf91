"""Throughput of Kara's decode-time compression step on one MI355X.

One step = one kara_compress call (window scoring, Top-K, Token2Chunk and
paged compaction for every sequence of the batch) on a synthetic workload
resident in HBM.  Prints one JSON line:

  value      window tokens compressed per second (each window token counted
             once across all layers of the model slice) = n_seqs * W / step time
  roofline   the scoring kernel (the dominant one) against the bf16 MFMA peak,
             with algorithmic flops 2 * Hq * W * W * D per (sequence, layer);
             its duration is measured with HIP events recorded on the call's
             stream around that kernel inside the timed steps
  cpu_baseline  the CPU oracle timed on a bounded sample of the same workload
                on all host threads (cpu_baseline_1core: one thread, smaller sample)
  parity     every unit's selection replayed by the oracle on the GPU's own
             float32 scores, and the sampled units of cpu_baseline against the
             float64 oracle (exact / near-tie accepted / failed)
  measured_ceilings  the chip's own MFMA, VALU, interleaved and copy rates from
                the library's probes, and the kernels' times against them
  secondary  the Qwen3-4B-shaped batch (32 sequences x 36 layers, W=1024),
             timed after the main workload

The default workload is the largest single-GPU one: Qwen3-14B-shaped, 128
sequences x 40 layers, W=2048 (config 3).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--config 3]
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

PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_FP32_MFMA_TFLOPS = 157.3  # MI355X fp32 (the tiny fp32 workload)
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
METRIC = "window tokens compressed/sec per GPU (score+topK+chunk+compact); % MFMA & HBM peak"


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


SCORE_SOURCES = ("kara_score_resident.hip", "kara_score_kernel.hpp")


def kernel_source_hash(names=SCORE_SOURCES):
    """sha256 prefix of the scoring kernels' sources (both scorers)."""
    h = hashlib.sha256()
    for name in names:
        with open(os.path.join(ROOT, "decode_kv_cache_kara_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def score_path(wl, flags):
    """Which scorer the library runs for this workload (the selection rule of
    the library's kara_internal.hpp, restated) and its executed logits per
    (sequence, layer): 'resident' scores with the window's keys in registers
    (16-row query tiles, one extra tile of MFMAs at the end of each launch;
    blocks of up to 1024 keys, 128 x NT keys per workgroup), 'two-pass'
    recomputes the region's logits (64-key tiles)."""
    import torch

    W, C, G, Hq = wl.window, wl.region, wl.n_q_heads // wl.n_kv_heads, wl.n_q_heads
    rows = G * W
    resident = (wl.dtype == torch.bfloat16 and wl.head_dim == 128 and W <= 2048 and rows <= 16384
                and not flags & 1)
    if not resident:
        return "two-pass", W * (math.ceil(W / 64) * 64 + math.ceil(C / 64) * 64) * (Hq // G) * G

    def keys(n):       # keys a launch with n resident keys multiplies: 8 waves x 16 NT, NT in {2, 4, 6, 8}
        nt = -(-(-(-n // 8)) // 16)
        nt = 2 if nt <= 2 else 4 if nt <= 4 else 6 if nt <= 6 else 8
        return 8 * 16 * nt

    rows_exec = (-(-rows // 16) + 1) * 16
    if W <= 1024:
        k = keys(W)
    else:
        k = keys(W - 1024) + 1024 + keys(max(C - 1024, 1))
    return "resident", rows_exec * k * wl.n_kv_heads


def read_traffic(workload):
    """HBM bytes per launch of the scoring kernel from the committed counter
    summary, if it was taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", f"score_kernel_{workload}_pmc.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        d = json.load(f)
    if d.get("source_sha256_16") != kernel_source_hash():
        return None
    return d.get("hbm_bytes_per_launch")


def host_cores():
    """Cores this process may run on (its CPU affinity)."""
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:
        return os.cpu_count() or 1


def sample_workload(wl, seqs, layers):
    """Host float64 copies of the inputs of the sampled (sequence, layer)
    pairs as a self-contained small workload: window queries [n_s, n_l, W, Hq,
    D], a pool [n_l, 2, NB', Hkv, bs, D] holding only the blocks from each
    sampled sequence's boundary block to its end (ids renumbered), the
    renumbered tables and the lengths."""
    import numpy as np
    import torch

    bs, W = wl.block_size, wl.window
    lens = [int(x) for x in wl.lens.cpu().tolist()]
    table = wl.table.cpu().long()
    li = torch.tensor(layers, dtype=torch.long, device=wl.pool.device)
    ids, rows = [], []
    MB = 0
    for b in seqs:
        f0, f1 = (lens[b] - W) // bs, -(-lens[b] // bs)
        row = np.full(f1, -2, dtype=np.int64)
        for e in range(f0, f1):
            row[e] = len(ids)
            ids.append(int(table[b, e]))
        rows.append(row)
        MB = max(MB, f1)
    tab = np.full((len(seqs), MB), -1, dtype=np.int64)
    for i, row in enumerate(rows):
        tab[i, :len(row)] = row
    blk = torch.tensor(ids, dtype=torch.long, device=wl.pool.device)
    pool = wl.pool.index_select(0, li).index_select(2, blk).to("cpu", torch.float64).numpy()
    q = torch.stack([wl.q_window[b].index_select(0, li) for b in seqs]).to("cpu", torch.float64).numpy()
    return q, pool, tab, np.array([lens[b] for b in seqs], dtype=np.int64)


def cpu_baseline(wl, seqs, layers, flags=0, one_core=False, gpu=None):
    """The oracle's compress() (float64 scores, Top-K, Token2Chunk) timed on
    the sampled (sequence, layer) pairs of the benchmark's own workload,
    scaled to the metric's unit (window tokens of the whole model slice per
    second: a pair is 1 / n_layers of one sequence's window).  With the GPU's
    outputs for the same workload (`gpu`: host scores, candidates and kept
    sets of every unit), the sampled units' parity against this oracle run is
    counted: exact, near-tie accepted (tests/parity.py's rule at 1e-3) or
    failed, and the largest relative score difference; and every unit's
    selection is replayed by the oracle in float32 on the GPU's own scores."""
    import numpy as np
    from threadpoolctl import threadpool_info, threadpool_limits

    from oracle import kara_oracle as ko

    uni, chunks = bool(flags & 1), not (flags & 2)
    q, pool, tab, lens = sample_workload(wl, seqs, layers)
    units = [(i, j) for i in range(len(seqs)) for j in range(len(layers))]
    with threadpool_limits(limits=1 if one_core else None):
        t0 = time.perf_counter()
        res = ko.compress(q, pool, tab, lens, wl.window, wl.protect, wl.top_k, wl.budget, wl.block_size, [],
                          units=units, unidirectional=uni, chunks=chunks)
        dt = time.perf_counter() - t0
    value = len(units) / wl.n_layers * wl.window / dt
    blas = 1 if one_core else max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    out = {"value": value, "unit": "window tokens/s", "cores": int(blas), "host_cores": host_cores(),
           "kind": "oracle",
           "sample": (f"oracle compress() (float64 scores, Top-K, Token2Chunk) on {len(units)} (sequence, layer) "
                      f"pairs = {len(units) * wl.n_kv_heads} units of this workload (sequences {list(seqs)}, "
                      f"layers {list(layers)} of {wl.n_layers}), {dt:.1f} s with {blas} BLAS thread(s), scaled to "
                      f"window tokens of the whole {wl.n_layers}-layer slice")}
    if gpu is not None:
        sys.path.insert(0, os.path.join(ROOT, "tests"))
        from parity import adjudicate
        Hkv = wl.n_kv_heads
        counts = {"exact": 0, "near_tie": 0, "fail": 0}
        worst = 0.0
        for i, b in enumerate(seqs):
            for j, l in enumerate(layers):
                for h in range(Hkv):
                    u = (b * wl.n_layers + l) * Hkv + h
                    s = res["scores"][i, j, h]
                    worst = max(worst, float((np.abs(gpu["scores"][u] - s) / np.abs(s)).max()))
                    v = adjudicate(s, wl.top_k, wl.budget, gpu["kept"][u], gpu["cand"][u], chunks=chunks)
                    counts["fail" if v.startswith("fail") else v] += 1
        out["parity"] = dict(counts, units=len(units) * Hkv, max_score_rel_err=worst)
        if not one_core:
            out["replay_all_units"] = replay_parity(wl, gpu, flags)
    return out


def replay_parity(wl, gpu, flags=0):
    """Every unit's selection replayed by the oracle in float32 on the GPU's
    own float32 scores (CPU worker processes); counts the units that differ
    (the bar is zero)."""
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    from parity import replay_mismatches
    t0 = time.perf_counter()
    bad = replay_mismatches(gpu["scores"], gpu["cand"], gpu["kept"], wl.top_k, wl.budget, chunks=not (flags & 2))
    return {"units": int(gpu["scores"].shape[0]), "mismatches": len(bad), "first": bad[:8],
            "seconds": round(time.perf_counter() - t0, 1)}


def measured_ceilings(score_ms, exec_flop, exec_logits, compact_ms, compact_bytes):
    """The chip's own ceilings for the scoring kernel's and the compaction's
    kinds of work, from the library's probes (MFMA loop, per-logit VALU loop,
    the two interleaved as in the scoring kernel's inner loop, streaming copy),
    each timed with HIP events on its launch stream after one warm-up launch,
    and the times those rates give for this launch's executed work."""
    import torch

    from decode_kv_cache_kara_amd import kara

    stream = torch.cuda.current_stream()
    scratch = torch.empty(kara.kara_probe_scratch_bytes() // 4, dtype=torch.float32, device="cuda")
    n = 4 << 30
    src = torch.ones(n // 4, dtype=torch.int32, device="cuda")
    dst = torch.empty_like(src)

    sink = torch.zeros(1, dtype=torch.int32, device="cuda")

    def rate(kind, iters, launches):
        kw = {"src": src} if kind in (kara.KARA_PROBE_COPY, kara.KARA_PROBE_READ) else {}
        out_t = {kara.KARA_PROBE_COPY: dst, kara.KARA_PROBE_READ: sink, kara.KARA_PROBE_WRITE: dst}.get(kind, scratch)
        kara.kara_probe(kind, iters, out_t, stream=stream, **kw)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        work = sum(kara.kara_probe(kind, iters, out_t, stream=stream, **kw) for _ in range(launches))
        e1.record(stream)
        torch.cuda.synchronize()
        return work / (e0.elapsed_time(e1) / 1e3)

    mfma = rate(kara.KARA_PROBE_MFMA, 100000, 3)          # flop/s
    valu = rate(kara.KARA_PROBE_VALU, 50000, 3)           # elements/s
    mix = rate(kara.KARA_PROBE_MIX, 10000, 3)             # logits/s
    copy = rate(kara.KARA_PROBE_COPY, 1, 3)               # bytes/s (read + written)
    read = rate(kara.KARA_PROBE_READ, 1, 3)               # bytes/s
    write = rate(kara.KARA_PROBE_WRITE, 1, 3)             # bytes/s
    del src, dst, scratch, sink
    bound_ms = exec_logits / mix * 1e3
    return {
        "mfma_bf16_tflops": round(mfma / 1e12, 1),
        "valu_softmax_gelem_per_s": round(valu / 1e9, 1),
        "mix_glogits_per_s": round(mix / 1e9, 1),
        "copy_gbs": round(copy / 1e9, 1),
        "read_gbs": round(read / 1e9, 1),
        "write_gbs": round(write / 1e9, 1),
        "score_kernel": {
            "executed_logits_per_launch": exec_logits,
            "mfma_alone_ms": round(exec_flop / mfma * 1e3, 3),
            "valu_alone_ms": round(exec_logits / valu * 1e3, 3),
            "interleaved_ms": round(bound_ms, 3),
            "measured_ms": round(score_ms, 3),
            "frac_of_interleaved": round(bound_ms / score_ms, 4),
        },
        "compact_kernel": {"copy_ms": round(compact_bytes / copy * 1e3, 3), "measured_ms": round(compact_ms, 3),
                           "frac_of_copy": round(compact_bytes / copy / (compact_ms / 1e3), 4)},
        "note": ("probes of this library (include/kara.h, kara_probe) run on the same GPU after the timed steps; "
                 "interleaved = the scoring kernel's inner loop (2*D MFMA flops and one multiply-add, exp2 and "
                 "add per logit) without memory traffic"),
    }


def _probe_note(da):
    if "paged_read_probe_gbs" not in da:
        return ""
    return f"; its loads alone {da['paged_read_probe_gbs']:.0f} GB/s ({da['frac_of_paged_read']:.1%} of them)"


def paged_read_ceiling(shape, layers, pool, table_d, lens_h, lens_d, attention_gbs, stream, launches=20):
    """The same launches' loads alone (kara_probe_paged_read: the attention
    kernel's workgroups, block-id staging and 16-byte K and V row loads, no
    arithmetic), cycling through `layers`; returns the probe's rate and the
    attention kernel's rate as a fraction of it."""
    import torch

    from decode_kv_cache_kara_amd import kara

    dst = torch.zeros(1, dtype=torch.int32, device="cuda")
    for k in range(3):
        kara.kara_probe_paged_read(shape, k % layers, pool, table_d, lens_h, lens_d, dst, stream=stream)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    nbytes = 0.0
    for k in range(launches):
        nbytes = kara.kara_probe_paged_read(shape, k % layers, pool, table_d, lens_h, lens_d, dst, stream=stream)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / launches
    gbs = nbytes / (ms / 1e3) / 1e9
    return {"paged_read_probe_gbs": round(gbs, 1), "paged_read_probe_ms": round(ms, 4),
            "frac_of_paged_read": round(attention_gbs / gbs, 4)}


def decode_attention_roofline(ses, wl, launches=36):
    """Decode attention over the cache as the last compression step left it
    (new tables and lengths): HBM bytes per launch = K and V rows of every
    cached token of one layer, averaged over `launches` launches that cycle
    through the layers; timed with HIP events on the launch stream."""
    import torch

    from decode_kv_cache_kara_amd import kara

    S, Hq, D, Lyr = wl.n_seqs, wl.n_q_heads, wl.head_dim, wl.n_layers
    lens_h = ses.new_lens_h.clone()
    lens_d = lens_h.cuda()
    table_d = ses.new_table_d
    g = torch.Generator(device="cuda").manual_seed(99)
    q = (torch.randn((S, Hq, D), generator=g, device="cuda") * 0.1).to(wl.dtype)
    out = torch.empty((S, Hq, D), device="cuda")
    ws = torch.empty(kara.kara_attention_workspace_bytes(ses.shape, S, int(lens_h.max())), dtype=torch.uint8,
                     device="cuda")
    stream = torch.cuda.current_stream()
    for l in range(3):
        kara.kara_decode_attention(ses.shape, l % Lyr, q, wl.pool, table_d, lens_h, lens_d, out, ws, stream=stream)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for k in range(launches):
        kara.kara_decode_attention(ses.shape, k % Lyr, q, wl.pool, table_d, lens_h, lens_d, out, ws, stream=stream)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / launches
    tokens = int(lens_h.sum())
    nbytes = 2.0 * tokens * wl.n_kv_heads * D * wl.pool.element_size()
    gbs = nbytes / (ms / 1e3) / 1e9
    res = {"bound": "hbm", "kernel": "attention_kernel+combine_kernel", "achieved": round(gbs, 1),
           "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4),
           "ms_per_launch": round(ms, 4), "algorithmic_bytes_per_launch": nbytes,
           "cached_tokens": tokens, "note": "one layer of all sequences over the compacted cache"}
    if wl.dtype == torch.bfloat16:
        res.update(paged_read_ceiling(ses.shape, Lyr, wl.pool, table_d, lens_h, lens_d, gbs, stream))
    return res


def decode_attention_one_layer(wl, lens_h, launches=20):
    """Decode attention over a one-layer cache of the workload's shape at the
    given (compacted) lengths, every block materialised: random bf16 K and V,
    each sequence's table a slice of a seeded permutation of the blocks.  For
    workloads whose prefix blocks are not materialised (the whole Qwen3-14B
    cache would not fit), one layer of it does (decode attention reads one
    layer per launch).  HBM bytes per launch = K and V rows of every cached
    token; timed with HIP events on the launch stream."""
    import numpy as np
    import torch

    from decode_kv_cache_kara_amd import kara

    S, Hq, Hkv, D, bs = wl.n_seqs, wl.n_q_heads, wl.n_kv_heads, wl.head_dim, wl.block_size
    lens = np.asarray(lens_h.cpu().numpy(), dtype=np.int64)
    nblk = (lens + bs - 1) // bs
    NB, MB = int(nblk.sum()), int(nblk.max())
    g = torch.Generator(device="cuda").manual_seed(7)
    pool = torch.empty((1, 2, NB, Hkv, bs, D), dtype=wl.dtype, device="cuda")
    pool.normal_(generator=g)
    perm = np.random.default_rng(7).permutation(NB).astype(np.int32)
    table = np.full((S, MB), -1, dtype=np.int32)
    off = np.concatenate([[0], np.cumsum(nblk)])
    for b in range(S):
        table[b, :nblk[b]] = perm[off[b]:off[b + 1]]
    table_d = torch.from_numpy(table).cuda()
    lens_h32 = torch.from_numpy(lens.astype(np.int32))
    lens_d = lens_h32.cuda()
    shape = kara.kara_shape(1, Hq, Hkv, D, bs, kara.dtype_code(wl.dtype))
    q = (torch.randn((S, Hq, D), generator=g, device="cuda") * 0.1).to(wl.dtype)
    out = torch.empty((S, Hq, D), device="cuda")
    ws = torch.empty(kara.kara_attention_workspace_bytes(shape, S, int(lens.max())), dtype=torch.uint8,
                     device="cuda")
    stream = torch.cuda.current_stream()
    for _ in range(3):
        kara.kara_decode_attention(shape, 0, q, pool, table_d, lens_h32, lens_d, out, ws, stream=stream)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(launches):
        kara.kara_decode_attention(shape, 0, q, pool, table_d, lens_h32, lens_d, out, ws, stream=stream)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / launches
    tokens = int(lens.sum())
    nbytes = 2.0 * tokens * Hkv * D * pool.element_size()
    gbs = nbytes / (ms / 1e3) / 1e9
    res = {"bound": "hbm", "kernel": "attention_kernel+combine_kernel", "achieved": round(gbs, 1),
           "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4),
           "ms_per_launch": round(ms, 4), "algorithmic_bytes_per_launch": nbytes,
           "cached_tokens": tokens,
           "note": ("one layer of the workload's shape at the lengths the compression step left, every block "
                    f"materialised with random values ({NB} blocks, {nbytes / 2**30:.1f} GiB), fragmented tables")}
    if wl.dtype == torch.bfloat16:
        res.update(paged_read_ceiling(shape, 1, pool, table_d, lens_h32, lens_d, gbs, stream))
    del pool
    torch.cuda.empty_cache()
    return res


def policy_sim(out, wl):
    """Periodic vs threshold vs no compression on the native serving
    simulator, with per-step costs from this run's measurements scaled to
    Distill-Llama-8B (32 layers, 8 KV heads of 128, like the measured slice):
    decode attention per cached token from `decode_attention`, one
    sequence's compression from the step time; the fixed per-step part
    (reading 16 GB of bf16 weights at 8 TB/s, 2 ms) is an assumption."""
    from decode_kv_cache_kara_amd import policy

    layers = 32
    att = out["decode_attention"]
    per_token = att["ms_per_launch"] / att["cached_tokens"] * layers
    per_seq = out["ms_per_step"] / wl.n_seqs * layers / wl.n_layers
    costs = dict(decode_ms_fixed=2.0, decode_ms_per_token=per_token, compress_ms_per_seq=per_seq,
                 compress_ms_per_key=per_seq / wl.window)
    rows = []
    for pol, mb, sm in policy.compare(costs):
        rows.append({"policy": pol, "max_batch": mb, "tokens_per_s": round(sm["tokens_per_s"], 1),
                     "compressions": sm["compressions"], "compress_share": round(sm["compress_share"], 5),
                     "preemptions": sm["preemptions"], "mean_running": round(sm["mean_active"], 1)})
    best = {p: max((r for r in rows if r["policy"] == p), key=lambda r: r["tokens_per_s"]) for p in
            ("periodic", "threshold", "none")}
    log("policy sim (best tokens/s): " + ", ".join(f"{p} {b['tokens_per_s']:.0f} at batch {b['max_batch']}"
                                                   for p, b in best.items()))
    return {"costs_ms": {k: float(f"{v:.6g}") for k, v in costs.items()}, "workload": policy.WORKLOAD,
            "rows": rows}


def run_trace(args, out_base):
    """Config 4: the periodic-compression serving trace.  A step is one
    compression event's kara_compress call; `--warmup` events run untimed,
    then up to `--steps` events (0: all remaining) are timed with HIP events
    around each call's kernels."""
    import torch

    from decode_kv_cache_kara_amd.trace import ServingTrace, TraceConfig

    cfg = TraceConfig()
    t0 = time.time()
    tr = ServingTrace(cfg)
    torch.cuda.synchronize()
    log(f"trace: {cfg.n_seqs} seqs x {cfg.n_layers} layers, {tr.n_events} events, pool {tr.NB} blocks "
        f"({tr.pool.numel() * 2 / 2**30:.1f} GiB), set up in {time.time() - t0:.1f} s")
    stream = torch.cuda.current_stream()
    calls = []
    n_warm = 0
    t_start = time.time()
    while not tr.done():
        batch = tr.next_event()
        if not batch:
            continue
        q = tr.window_queries(batch)
        if n_warm < args.warmup:
            tr.compress(batch, q, stream=stream)
            n_warm += 1
            continue
        if args.steps and len(calls) >= args.steps:
            tr.compress(batch, q, stream=stream)
            continue
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
        for e in ev:
            e.record(stream)
        torch.cuda.synchronize()
        tr.compress(batch, q, stream=stream, stage_events=[e.cuda_event for e in ev])
        calls.append((len(batch), ev))
        if len(calls) % 20 == 0:
            log(f"event {tr.events}: {len(calls)} timed calls, {time.time() - t_start:.0f} s")
    torch.cuda.synchronize()
    total_ms = sum(ev[0].elapsed_time(ev[3]) for _, ev in calls)
    stage = [sum(ev[i].elapsed_time(ev[i + 1]) for _, ev in calls) for i in range(3)]
    n_comp = sum(n for n, _ in calls)
    W = cfg.window
    value = n_comp * W / (total_ms / 1e3)
    score_flop = 2.0 * n_comp * cfg.n_layers * cfg.n_q_heads * W * W * cfg.head_dim
    score_tflops = score_flop / (stage[0] / 1e3) / 1e12
    # the trace's caches are bf16: the scorer is chosen by head size, window and rows
    resident = cfg.head_dim == 128 and W <= 2048 and cfg.n_q_heads // cfg.n_kv_heads * W <= 16384
    log(f"{len(calls)} timed calls, {n_comp} sequence compressions, {total_ms:.1f} ms total")
    out = dict(out_base)
    out.update({
        "value": round(value, 1),
        "steps": len(calls),
        "warmup": n_warm,
        "ms_per_step": round(total_ms / max(len(calls), 1), 4),
        "data": "synthetic serving trace (seeded decode appends with planted spans, 50% random selection per event)",
        "config": {"workload": "distill-llama-8b-periodic-trace", "n_seqs": cfg.n_seqs,
                   "n_layers": cfg.n_layers, "n_q_heads": cfg.n_q_heads, "n_kv_heads": cfg.n_kv_heads,
                   "head_dim": cfg.head_dim, "window": W, "protect": cfg.protect, "top_k": cfg.top_k,
                   "budget": cfg.budget, "period": cfg.period, "lengths": f"{cfg.init_len}->{cfg.max_len}",
                   "events": tr.events, "compressions_timed": n_comp},
        "roofline": {"bound": "mfma",
                     "kernel": ("score_resident_kernel + exact_resident_kernel (marked units only)" if resident
                                else "score_kernel"),
                     "achieved": round(score_tflops, 2),
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": round(score_tflops / PEAK_BF16_TFLOPS, 4),
                     "traffic": None, "algorithmic_flop_total": score_flop,
                     "scorer": "resident" if resident else "two-pass",
                     "kernel_source_sha256_16": kernel_source_hash()},
        "stages_ms": {"score": round(stage[0], 3), "select": round(stage[1], 3), "compact": round(stage[2], 3)},
    })
    return out


def run_batch(cfg, args, flags, steps, warmup, extras=True, keep_outputs=False):
    """Times `steps` kara_compress calls on one synthetic workload (inputs
    resident in HBM; `warmup` untimed calls first) and returns the report
    fields, the workload and, with keep_outputs, host copies of one further
    call's scores, candidates and kept sets."""
    import torch

    from decode_kv_cache_kara_amd import kara, runner, synth

    t0 = time.time()
    wl = synth.make_workload(cfg, seed=args.seed, device="cuda")
    torch.cuda.synchronize()
    log(f"workload {wl.name}: {wl.n_seqs} seqs x {wl.n_layers} layers, pool {wl.n_blocks} blocks "
        f"({wl.pool.numel() * wl.pool.element_size() / 2**30:.1f} GiB), generated in {time.time() - t0:.1f} s")
    ses = runner.Session(wl, outputs=False, flags=flags)
    stream = torch.cuda.current_stream()

    def events():
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
        for e in ev:
            e.record(stream)      # materialise the handles
        return ev

    for _ in range(warmup):
        ses.compress(stream=stream)
    torch.cuda.synchronize()
    log(f"warmup done ({warmup} steps)")

    step_events = [events() for _ in range(steps)]
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for k in range(steps):
        ses.compress(stream=stream, stage_events=[e.cuda_event for e in step_events[k]])
    stop.record(stream)
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(stop)
    ms_per_step = total_ms / steps
    stage = [0.0, 0.0, 0.0]
    for ev in step_events:
        for i in range(3):
            stage[i] += ev[i].elapsed_time(ev[i + 1])
    stage = [x / steps for x in stage]
    per_step = sorted(ev[0].elapsed_time(ev[3]) for ev in step_events)
    log(f"timed {steps} steps: {ms_per_step:.3f} ms/step; score {stage[0]:.3f} ms, "
        f"select {stage[1]:.3f} ms, compact {stage[2]:.3f} ms")

    S, Lyr, Hq, Hkv, D, W, C = (wl.n_seqs, wl.n_layers, wl.n_q_heads, wl.n_kv_heads, wl.head_dim,
                                wl.window, wl.region)
    elt = wl.pool.element_size()
    tokens = S * W
    value = tokens / (ms_per_step / 1e3)
    uni = bool(flags & kara.UNIDIRECTIONAL)
    # one QK^T over the window: all W x W logits, or (unidirectional) the
    # W (W + 1) / 2 that causal attention needs
    score_flop = 2.0 * S * Lyr * Hq * (W * (W + 1) / 2 if uni else W * W) * D
    path, exec_logits_sl = score_path(wl, flags)
    exec_flop = 2.0 * S * Lyr * exec_logits_sl * D
    score_tflops = score_flop / (stage[0] / 1e3) / 1e12
    peak = PEAK_BF16_TFLOPS if wl.dtype == torch.bfloat16 else PEAK_FP32_MFMA_TFLOPS
    lens = ses.lens_h.tolist()
    rows = sum(((L - W) % wl.block_size) + wl.budget + wl.protect for L in lens)
    compact_bytes = 2.0 * rows * Lyr * 2 * Hkv * D * elt
    compact_gbs = compact_bytes / (stage[2] / 1e3) / 1e9
    traffic = read_traffic(wl.name) if flags == 0 else None
    materialized = not bool((wl.table == -2).any())

    out = {
        "value": round(value, 1),
        "token_layers_per_s": round(value * Lyr, 1),
        "ms_per_step": round(ms_per_step, 4),
        "dtype": "bf16" if wl.dtype == torch.bfloat16 else "f32",
        "config": {"workload": wl.name, "n_seqs": S, "n_layers": Lyr, "n_q_heads": Hq, "n_kv_heads": Hkv,
                   "head_dim": D, "window": W, "protect": wl.protect, "top_k": wl.top_k,
                   "budget": wl.budget, "block_size": wl.block_size,
                   "seq_lens": f"U[{min(lens)}..{max(lens)}] seed {wl.seed}",
                   "prefix_blocks": "materialised" if materialized else
                   "not materialised (table entries before the boundary block are never read by the step)",
                   "ablation": {0: "none", 1: "unidirectional", 2: "no_chunks", 3: "unidirectional+no_chunks"}[flags]},
        "roofline": {"bound": "mfma",
                     "kernel": (("score_resident_kernel (3 launches)" if W > 1024 else
                                 "score_resident_kernel + exact_resident_kernel (marked units only)")
                                if path == "resident" else "score_kernel"),
                     "achieved": round(score_tflops, 2),
                     "peak": peak, "unit": "TFLOP/s", "frac": round(score_tflops / peak, 4),
                     "traffic": traffic, "algorithmic_flop_per_launch": score_flop,
                     "executed_mfma_flop_per_launch": exec_flop if not uni else None,
                     "executed_frac": (round(exec_flop / (stage[0] / 1e3) / 1e12 / peak, 4) if not uni else None),
                     "scorer": path, "kernel_source_sha256_16": kernel_source_hash()},
        "stages_ms": {"score": round(stage[0], 4), "select": round(stage[1], 4),
                      "compact": round(stage[2], 4)},
        "kernel_ms_per_step": {"median": round(per_step[len(per_step) // 2], 4), "min": round(per_step[0], 4),
                               "max": round(per_step[-1], 4)},
        "compact_roofline": {"bound": "hbm", "kernel": "compact_kernel", "achieved": round(compact_gbs, 1),
                             "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(compact_gbs / PEAK_HBM_GBS, 4),
                             "algorithmic_bytes_per_launch": compact_bytes},
    }
    if extras and materialized:
        out["decode_attention"] = decode_attention_roofline(ses, wl)
        log(f"decode attention over the compacted cache: {out['decode_attention']['ms_per_launch']:.3f} ms/layer, "
            f"{out['decode_attention']['achieved']:.0f} GB/s{_probe_note(out['decode_attention'])}")
    elif extras:
        out["decode_attention"] = decode_attention_one_layer(wl, ses.new_lens_h)
        log(f"decode attention over a one-layer cache at the compacted lengths: "
            f"{out['decode_attention']['ms_per_launch']:.3f} ms/layer, {out['decode_attention']['achieved']:.0f} GB/s"
            f"{_probe_note(out['decode_attention'])}")
    if extras and wl.dtype == torch.bfloat16 and not uni:
        exec_logits = exec_flop / (2.0 * D)
        out["measured_ceilings"] = measured_ceilings(stage[0], exec_flop, exec_logits, stage[2], compact_bytes)
        mc = out["measured_ceilings"]
        log(f"measured ceilings: MFMA {mc['mfma_bf16_tflops']} TFLOP/s, softmax VALU {mc['valu_softmax_gelem_per_s']} "
            f"Gelem/s, interleaved {mc['mix_glogits_per_s']} Glogit/s, copy {mc['copy_gbs']} GB/s (read "
            f"{mc['read_gbs']}, write {mc['write_gbs']}); score kernel at "
            f"{mc['score_kernel']['frac_of_interleaved']:.1%} of its interleaved bound")
    gpu = None
    if keep_outputs:
        outs = runner.Session(wl, outputs=True, flags=flags)
        outs.compress(stream=stream)
        torch.cuda.synchronize()
        gpu = {"scores": outs.scores.cpu().numpy(), "cand": outs.cand.cpu().numpy(),
               "kept": outs.retained.cpu().numpy()}
        del outs
    del ses
    return out, wl, gpu


def spread(n, k):
    """k indices spread over range(n), the first and the last included."""
    if k >= n:
        return list(range(n))
    return sorted({round(i * (n - 1) / (k - 1)) for i in range(k)})


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None,
                    help="timed steps (default 20; for the trace, all events after warmup)")
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", type=int, default=3, choices=[0, 1, 2, 3, 4],
                    help="workload (default 3: Qwen3-14B-shaped, 128 sequences x 40 layers, W=2048)")
    ap.add_argument("--seed", type=int, default=None)
    ap.add_argument("--flags", type=int, default=0, choices=[0, 1, 2, 3],
                    help="ablations: 1 unidirectional scoring, 2 Token2Chunk off, 3 both")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-secondary", action="store_true",
                    help="skip the Qwen3-4B-shaped batch measured after the main workload")
    ap.add_argument("--no-extras", action="store_true",
                    help="time the step only (no decode attention, probes or policy simulation)")
    ap.add_argument("--cpu-pairs", type=str, default="4x8",
                    help="oracle sample: sequences x layers of the workload (default 4x8 = 32 pairs)")
    ap.add_argument("--copy-calibration", type=float, default=0.0, metavar="GIB",
                    help="only run a device-to-device copy of this many GiB three times (the reference "
                         "kernel that scales the HBM byte counters) and print its size")
    args = ap.parse_args()
    if args.steps is None:
        args.steps = 0 if args.config == 4 else 20

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures the compression step on one GPU only; --gpus must be 1 "
              "(every unit of work is independent, so more GPUs would each run their own batch).",
              file=sys.stderr)
        sys.exit(2)

    import torch

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)

    if args.copy_calibration:
        n = int(args.copy_calibration * 2**30)
        src = torch.ones(n // 4, dtype=torch.int32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_per_launch": n, "launches": 3}), flush=True)
        return

    base = {"metric": METRIC, "unit": "window tokens/s", "n_gpus": 1, "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": "bf16"}
    if args.config == 4:
        out = run_trace(args, base)
        print(json.dumps(out), flush=True)
        return

    res, wl, gpu = run_batch(args.config, args, args.flags, args.steps, args.warmup, extras=not args.no_extras,
                             keep_outputs=not args.no_cpu_baseline)
    out = dict(base)
    out.update({"value": res.pop("value"), "steps": args.steps, "warmup": args.warmup,
                "ms_per_step": res.pop("ms_per_step"), "dtype": res.pop("dtype"),
                "data": "synthetic (seeded Gaussian Q/K/V; planted spans where the workload has them; fragmented "
                        "block tables)",
                "config": res.pop("config")})
    out.update(res)
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a sample of the same workload ...")
        n_s, n_l = (int(x) for x in args.cpu_pairs.split("x"))
        seqs, layers = spread(wl.n_seqs, n_s), spread(wl.n_layers, n_l)
        out["cpu_baseline"] = cpu_baseline(wl, seqs, layers, flags=args.flags, gpu=gpu)
        log(f"cpu baseline {out['cpu_baseline']['value']:.1f} window tokens/s; sampled parity "
            f"{out['cpu_baseline']['parity']}")
        out["cpu_baseline_1core"] = cpu_baseline(wl, seqs[:1], layers[:1], flags=args.flags, one_core=True)
        log(f"cpu baseline on one core {out['cpu_baseline_1core']['value']:.1f} window tokens/s")
        out["parity"] = {"replay_all_units": out["cpu_baseline"].pop("replay_all_units"),
                         "sampled_vs_float64_oracle": out["cpu_baseline"]["parity"],
                         "rule": "scores within 1e-3 relative; selection replayed in float32 on the GPU's scores "
                                 "bit-exact for every unit; sampled units exact or near-ties within 1e-3"}
        log(f"replay of every unit: {out['parity']['replay_all_units']}")
    if args.config == 2 and args.flags == 0 and not args.no_extras:
        out["policy_sim"] = policy_sim(out, wl)
    del wl, gpu
    torch.cuda.empty_cache()
    if args.config == 3 and not args.no_secondary:
        sec, wl2, _ = run_batch(2, args, args.flags, max(10, args.steps // 2), args.warmup,
                                extras=not args.no_extras)
        out["secondary"] = sec
        if args.flags == 0 and not args.no_extras:
            out["policy_sim"] = policy_sim(sec, wl2)
        del wl2
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
