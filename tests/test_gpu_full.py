"""GPU parity at full workload sizes, in the launch configuration bench.py
times: Qwen3-4B 36-layer batch 32 (all blocks materialised), Qwen3-14B
40-layer batch 128 (window and boundary blocks materialised), and one event of
the Distill-Llama-8B-shaped trace as a static batch.  The selection of every
unit is replayed by the oracle on the GPU's own float32 scores and must match
bit for bit; the float64 oracle scores sampled (sequence, layer) pairs on the
exact bytes the kernels read (at least 256 units per workload, each sampled
sequence at its first and last layer); bookkeeping (tables, lengths, free list) is checked for every sequence, and
per-block checksums show that no block other than the fresh ones changed.
The Qwen3-4B batch also runs with both ablations switched on (unidirectional
scoring, Token2Chunk off)."""

import numpy as np
import pytest
import torch

from oracle import kara_oracle as ko
from parity import adjudicate, assert_scores_close, oracle_scores_many, replay_selection, tally

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from decode_kv_cache_kara_amd import runner, synth


def block_checksums(pool):
    """Per-block int64 sum of the 32-bit words of every layer, K and V."""
    Lyr, _, NB = pool.shape[:3]
    w = pool.view(torch.int32) if pool.dtype == torch.float32 else pool.view(torch.int16)
    out = torch.zeros(NB, dtype=torch.int64, device=pool.device)
    for l in range(Lyr):
        for kv in range(2):
            out += w[l, kv].reshape(NB, -1).sum(dim=1, dtype=torch.int64)
    return out


def gather_rows(pool, table_row, tokens, l, kv, bs):
    t = torch.tensor(tokens, dtype=torch.long, device=pool.device)
    blk = table_row.to(pool.device).long()[t // bs]
    return pool[l, kv, blk, :, t % bs, :]          # [n, Hkv, D]


def sample_pairs(cfg, S, Lyr):
    """(sequence, layer) pairs whose units the float64 oracle scores: every
    sequence's first and last layer (Qwen3-4B batch: 64 pairs, 512 units;
    Qwen3-14B batch: 256 pairs, 2048 units, a few minutes of CPU work in the
    worker processes; trace event: 32 pairs, 256 units)."""
    return [(b, l) for b in range(S) for l in sorted({0, Lyr - 1})]


@pytest.mark.timeout(1200)
@pytest.mark.parametrize("cfg,flags", [(2, 0), (3, 0), (4, 0), (2, 3)])
def test_full_size_sampled(cfg, flags):
    print(f"[case] full size config {cfg} flags {flags}", flush=True)
    uni, chunks = bool(flags & 1), not (flags & 2)
    wl = synth.make_workload(cfg, device="cuda")
    torch.cuda.synchronize()
    ses = runner.Session(wl, flags=flags)
    S, Lyr, W, B, bs = wl.n_seqs, wl.n_layers, wl.window, wl.protect, wl.block_size
    samples = sample_pairs(cfg, S, Lyr)
    if flags:
        samples = samples[:: max(1, len(samples) // 16)]
    lens = ses.lens_h.numpy().astype(np.int64)
    table = ses.table_h
    snap = {}
    for b, l in samples:
        L = int(lens[b])
        f0 = (L - W) // bs
        tail = list(range(f0 * bs, L))
        snap[b, l] = dict(
            q=wl.q_window[b, l].float().cpu().numpy(),
            k=gather_rows(wl.pool, table[b], list(range(L - W, L)), l, 0, bs).float().cpu().numpy(),
            tail=[gather_rows(wl.pool, table[b], tail, l, kv, bs).cpu() for kv in range(2)])
    sums_before = block_checksums(wl.pool)
    pool = ses.compress()
    torch.cuda.synchronize()
    print(f"[case] config {cfg} compressed; checking {len(samples)} sampled pairs", flush=True)

    # bookkeeping of every sequence
    fifo = ko.FifoPool(wl.free_ids)
    new_table, new_lens = ko.plan_compaction(table.numpy().astype(np.int64), lens, W, B, wl.budget, bs, fifo)
    assert ses.new_table_h.numpy().tolist() == new_table.tolist()
    assert ses.new_lens_h.numpy().tolist() == new_lens.tolist()
    assert pool.snapshot() == fifo.ids()
    fresh = sorted({int(x) for row in new_table for x in row if x >= 0}
                   - {int(x) for x in table.numpy().ravel() if x >= 0})
    sums_after = block_checksums(wl.pool)
    keep = torch.ones(wl.n_blocks, dtype=torch.bool, device="cuda")
    keep[torch.tensor(fresh, dtype=torch.long, device="cuda")] = False
    assert torch.equal(sums_before[keep], sums_after[keep])

    # selection of every unit replayed on the GPU's own float32 scores
    gs_all = ses.scores.cpu().numpy()
    cand_all = ses.cand.cpu().numpy()
    kept_all = ses.retained.cpu().numpy()
    replayed = replay_selection(gs_all, cand_all, kept_all, wl.top_k, wl.budget, chunks=chunks)
    print(f"[case] config {cfg}: {replayed} units replayed bit-exact", flush=True)

    Hkv = wl.n_kv_heads
    scores = gs_all.reshape(S, Lyr, Hkv, -1)
    cand = cand_all.reshape(S, Lyr, Hkv, -1)
    kept = kept_all.reshape(S, Lyr, Hkv, -1)
    orc = oracle_scores_many([(snap[p]["q"], snap[p]["k"]) for p in samples], B, unidirectional=uni,
                             label=f"config {cfg}")
    verdicts = {}
    worst = 0.0
    for (b, l), s in zip(samples, orc):
        worst = max(worst, assert_scores_close(scores[b, l], s, what=f"scores of ({b},{l})"))
        for h in range(Hkv):
            v = adjudicate(s[h], wl.top_k, wl.budget, kept[b, l, h], cand[b, l, h], chunks=chunks)
            assert not v.startswith("fail"), (b, l, h, v)
            verdicts[v] = verdicts.get(v, 0) + 1
        # compacted rows: the boundary block's leading tokens, the kept tokens, the protected tokens
        L = int(lens[b])
        start = L - W
        f0 = start // bs
        p = start - f0 * bs
        n_new = p + wl.budget + B
        new_rows = [gather_rows(wl.pool, ses.new_table_h[b], list(range(f0 * bs, f0 * bs + n_new)), l, kv, bs).cpu()
                    for kv in range(2)]
        for kv in range(2):
            old = snap[b, l]["tail"][kv]                       # rows of tokens f0*bs .. L-1
            for h in range(Hkv):
                idx = list(range(p)) + [p + int(j) for j in kept[b, l, h]] + list(range(p + W - B, p + W))
                want = old[idx, h]
                got = new_rows[kv][:, h]
                assert torch.equal(want.view(torch.int16) if want.dtype == torch.bfloat16 else want,
                                   got.view(torch.int16) if got.dtype == torch.bfloat16 else got)
    tally(f"full size {wl.name} flags {flags}", verdicts, worst, replayed)
    print(f"[case] config {cfg} verdicts {verdicts}, max score rel err {worst:.3g}", flush=True)


@pytest.fixture(autouse=True)
def _release_memory():
    yield
    import gc
    gc.collect()
    if torch.cuda.is_available():
        torch.cuda.empty_cache()
