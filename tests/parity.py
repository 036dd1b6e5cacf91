"""Helpers for comparing the HIP path with the CPU oracle.

The oracle always runs on the exact bytes the GPU consumed (copied back from
device memory) and never on anything the HIP path produced.  Where several
results are correct (selections decided by near-equal scores), the GPU result
is checked for validity against the oracle's scores instead of for equality.
"""

from __future__ import annotations

import math

import numpy as np
import torch

from oracle import kara_oracle as ko

SCORE_RTOL = 1e-3       # tolerance on the window scores (float32 accumulate vs float64)

# Per-case parity counts, printed at the end of the session (tests/conftest.py)
# and written as JSON where KARA_PARITY_REPORT names a file.
TALLY: dict = {}


def tally(case, verdicts=None, max_rel_err=None, replayed=0):
    """Adds one check's results to the session's per-case counts."""
    t = TALLY.setdefault(case, {"exact": 0, "near_tie": 0, "fail": 0, "replayed_bit_exact": 0,
                                "max_score_rel_err": 0.0})
    for v, n in (verdicts or {}).items():
        key = "fail" if v.startswith("fail") else v
        t[key] = t.get(key, 0) + n
    if max_rel_err is not None:
        t["max_score_rel_err"] = max(t["max_score_rel_err"], float(max_rel_err))
    t["replayed_bit_exact"] += int(replayed)
    return t


def _replay_chunk(args):
    """Worker: the oracle's Top-K and Token2Chunk on the GPU's own float32
    scores of a run of units; returns the units whose results differ."""
    gs, cand, kept, K, R, chunks, first = args
    bad = []
    for i in range(gs.shape[0]):
        if (cand[i].tolist() != ko.topk_candidates(gs[i], K).tolist()
                or kept[i].tolist() != ko.select_retained(gs[i], K, R, chunks=chunks).tolist()):
            bad.append(first + i)
    return bad


_POOL = None


def _one_blas_thread():
    """Worker initialiser: one BLAS thread per worker process, so that the
    workers together use each core once."""
    from threadpoolctl import threadpool_limits
    threadpool_limits(limits=1)


def cpu_workers():
    """CPU worker processes for large replays and oracle samples (spawned:
    they import NumPy and the oracle only and never touch the GPU), one per
    core this process may use, leaving one, with one BLAS thread each."""
    global _POOL
    if _POOL is None:
        import concurrent.futures
        import multiprocessing
        import os
        n = max(1, min(15, len(os.sched_getaffinity(0)) - 1))
        _POOL = concurrent.futures.ProcessPoolExecutor(max_workers=n, initializer=_one_blas_thread,
                                                       mp_context=multiprocessing.get_context("spawn"))
        import atexit
        atexit.register(_POOL.shutdown)
    return _POOL


def replay_mismatches(gpu_scores, cand, kept, K, R, chunks=True):
    """Units whose candidates or kept set differ from the oracle's Top-K and
    Token2Chunk run in float32 on the GPU's own float32 scores."""
    gs = np.ascontiguousarray(np.asarray(gpu_scores, dtype=np.float32))
    cand = np.asarray(cand)
    kept = np.asarray(kept)
    U = gs.shape[0]
    if U * gs.shape[1] <= 2_000_000:
        return _replay_chunk((gs, cand, kept, K, R, chunks, 0))
    step = max(64, U // 64)
    jobs = [(gs[a:a + step], cand[a:a + step], kept[a:a + step], K, R, chunks, a) for a in range(0, U, step)]
    return [u for part in cpu_workers().map(_replay_chunk, jobs) for u in part]


def replay_selection(gpu_scores, cand, kept, K, R, chunks=True):
    """Selection parity on the GPU's own scores: for every unit, the oracle's
    Top-K and Token2Chunk, run in float32 on the float32 scores the GPU
    produced, give exactly the GPU's candidates and kept set.  All decisions
    of these stages are comparisons and correctly rounded float32 operations,
    so nothing is left to tolerance.  Returns the number of units checked."""
    U = np.asarray(gpu_scores).shape[0]
    bad = replay_mismatches(gpu_scores, cand, kept, K, R, chunks)
    assert not bad, f"replay differs from the GPU on {len(bad)} of {U} units, first {bad[:8]}"
    return U


def host_inputs(wl):
    """Oracle-side copies of a workload's inputs: float64 states, int tables."""
    q = wl.q_window.detach().to("cpu", torch.float64).numpy()
    pool = wl.pool.detach().to("cpu", torch.float64).numpy()
    table = wl.table.detach().to("cpu", torch.int64).numpy()
    lens = wl.lens.detach().to("cpu", torch.int64).numpy()
    return q, pool, table, lens


def oracle_scores(wl, units=None, unidirectional=False):
    """float64 scores [S, Lyr, Hkv, C] (rows outside `units` stay NaN)."""
    q, pool, table, lens = host_inputs(wl)
    out = np.full((wl.n_seqs, wl.n_layers, wl.n_kv_heads, wl.region), np.nan)
    todo = units if units is not None else [(b, l) for b in range(wl.n_seqs) for l in range(wl.n_layers)]
    for b, l in todo:
        k = ko.window_keys(pool, table[b], int(lens[b]), wl.window, l, wl.n_kv_heads, wl.block_size)
        out[b, l] = ko.window_scores(q[b, l], k, wl.protect, unidirectional)
    return out


def assert_scores_close(gpu, orc, rtol=SCORE_RTOL, what="scores"):
    gpu = np.asarray(gpu, dtype=np.float64)
    orc = np.asarray(orc, dtype=np.float64)
    assert gpu.shape == orc.shape
    err = np.abs(gpu - orc)
    bad = err > rtol * np.abs(orc)
    if bad.any():
        i = np.unravel_index(np.argmax(err / np.maximum(np.abs(orc), 1e-30)), err.shape)
        raise AssertionError(f"{what}: {int(bad.sum())} of {bad.size} elements beyond rtol={rtol}; "
                             f"worst at {i}: gpu={gpu[i]!r} oracle={orc[i]!r}")
    return float((err / np.maximum(np.abs(orc), 1e-300)).max())


def _close(a, b, tol):
    return abs(a - b) <= tol * max(abs(a), abs(b))


def adjudicate(s, K, R, X, candX, tol=SCORE_RTOL, chunks=True):
    """Classify the GPU's kept set X and candidates candX of one unit against the
    oracle's float64 scores s: 'exact', 'near_tie' or 'fail: reason'.
    chunks=False judges the Token2Chunk-off ablation (X must be a top-R set).

    'exact' means both equal the oracle's own result.  'near_tie' means they
    differ from it but are a valid result of the method under some perturbation
    of the scores within `tol` (relative): the candidates are a top-K, the
    accepted spans are a prefix of the chunk-score order that stops at a span
    that does not fit, and the top-ups are the best remaining positions, each
    condition allowed to bend only between near-equal values.
    """
    s = np.asarray(s, dtype=np.float64)
    C = len(s)
    X = [int(x) for x in X]
    candX = [int(x) for x in candX]
    candY = ko.topk_candidates(s, K).tolist()
    Y = ko.select_retained(s, K, R, chunks=chunks).tolist()
    if len(X) != R or any(a >= b for a, b in zip(X, X[1:])) or X[0] < 0 or X[-1] >= C:
        return "fail: kept set malformed"
    if len(candX) != K or any(a >= b for a, b in zip(candX, candX[1:])) or candX[0] < 0 or candX[-1] >= C:
        return "fail: candidates malformed"
    if X == Y and candX == candY:
        return "exact"

    def best_of_rest_ok(chosen, pool_positions):
        rest = [j for j in pool_positions if j not in chosen]
        if not chosen or not rest:
            return True
        lo = min(s[j] for j in chosen)
        hi = max(s[j] for j in rest)
        return lo >= hi * (1 - tol) if hi > 0 else lo >= hi - tol * abs(hi)

    cx = set(candX)
    if not best_of_rest_ok(cx, range(C)):
        return "fail: candidates are not a top-K"
    Xs = set(X)
    if R < K or not chunks:
        if R >= K and not cx <= Xs:
            return "fail: candidates not kept"
        return "near_tie" if best_of_rest_ok(Xs, range(C)) else "fail: not a top-R set"
    if not cx <= Xs:
        return "fail: candidates not kept"
    spans = [((s[a] + s[b]) / (b - a + 1), a, b) for a, b in zip(candX[:-1], candX[1:]) if b - a > 1]
    acc = [t for t in spans if set(range(t[1] + 1, t[2])) <= Xs]
    rej = [t for t in spans if t not in acc]
    used = sum(b - a - 1 for _, a, b in acc)
    room = R - K
    if used > room:
        return "fail: spans exceed the budget"
    if acc and rej and min(t[0] for t in acc) < max(t[0] for t in rej) * (1 - tol):
        return "fail: a better span was passed over"
    if rej:
        top = max(t[0] for t in rej)
        if not any(t[0] >= top * (1 - tol) and (t[2] - t[1] - 1) > room - used for t in rej):
            return "fail: a fitting span was skipped"
    base = set(cx)
    for _, a, b in acc:
        base |= set(range(a + 1, b))
    tops = Xs - base
    if not best_of_rest_ok(tops, [j for j in range(C) if j not in base]):
        return "fail: top-up is not the best remaining"
    return "near_tie"


def expected_rows(wl_pool_cpu, table, lens, window, protect, block_size, kept, b, l, kv, h):
    """Old-cache rows that the compacted tail of (b, l, kv, h) must hold, in order."""
    L = int(lens[b])
    start = L - window
    f0 = start // block_size
    toks = (list(range(f0 * block_size, start)) + [start + int(j) for j in kept]
            + list(range(L - protect, L)))
    rows = [wl_pool_cpu[l, kv, int(table[b][t // block_size]), h, t % block_size] for t in toks]
    return torch.stack(rows) if rows else None


def tail_rows(pool_cpu, new_table, b, l, kv, h, f0, n, block_size):
    rows = []
    for i in range(n):
        pos = f0 * block_size + i
        rows.append(pool_cpu[l, kv, int(new_table[b][pos // block_size]), h, pos % block_size])
    return torch.stack(rows)


def bits(t):
    """Bit pattern view of a tensor for byte-exact comparisons."""
    if t.dtype in (torch.bfloat16, torch.float16):
        return t.view(torch.int16)
    if t.dtype == torch.float32:
        return t.view(torch.int32)
    return t


def _scores_job(args):
    q, k, protect, uni = args
    return ko.window_scores(q, k, protect, unidirectional=uni)


def oracle_scores_many(pairs, protect, unidirectional=False, label=None):
    """The oracle's float64 window scores for a list of (q_window, k_window)
    host arrays, computed in the CPU worker processes.  With a label, a
    progress line is printed about every 20 s while the results come in."""
    import concurrent.futures as cf
    import time
    jobs = [(q, k, protect, unidirectional) for q, k in pairs]
    if len(jobs) <= 2:
        return [_scores_job(j) for j in jobs]
    futs = [cpu_workers().submit(_scores_job, j) for j in jobs]
    if label:
        t0 = last = time.time()
        for n, _ in enumerate(cf.as_completed(futs), 1):
            if time.time() - last >= 20 or n == len(futs):
                last = time.time()
                print(f"[case] {label}: oracle scores {n}/{len(futs)} ({last - t0:.0f} s)", flush=True)
    return [f.result() for f in futs]


def pair_verdicts_job(args):
    """Worker: float64 oracle scores of one (sequence, layer) pair, their
    largest relative difference from the GPU's scores, and the verdicts of the
    GPU's kept sets against them (one per KV head)."""
    q, k, protect, top_k, budget, gpu_scores, cand, kept = args
    s = ko.window_scores(q, k, protect)
    err = float((np.abs(gpu_scores - s) / np.abs(s)).max())
    verdicts = [adjudicate(s[h], top_k, budget, kept[h], cand[h]) for h in range(s.shape[0])]
    return err, verdicts
