"""GPU parity at full workload sizes, in the launch configuration bench.py
times: Qwen3-4B 36-layer batch 32 (all blocks materialised), Qwen3-14B
40-layer batch 128 (window and boundary blocks materialised), and one event of
the Distill-Llama-8B-shaped trace as a static batch.  The oracle checks
sampled (sequence, layer) pairs one by one on the exact bytes the kernels read;
bookkeeping (tables, lengths, free list) is checked for every sequence, and
per-block checksums show that no block other than the fresh ones changed.
The Qwen3-4B batch also runs with both ablations switched on (unidirectional
scoring, Token2Chunk off)."""

import numpy as np
import pytest
import torch

from oracle import kara_oracle as ko
from parity import adjudicate, assert_scores_close

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


@pytest.mark.parametrize("cfg,flags", [(2, 0), (3, 0), (4, 0), (2, 3)])
def test_full_size_sampled(cfg, flags):
    print(f"[case] full size config {cfg} flags {flags}", flush=True)
    uni, chunks = bool(flags & 1), not (flags & 2)
    wl = synth.make_workload(cfg, device="cuda")
    torch.cuda.synchronize()
    ses = runner.Session(wl, flags=flags)
    S, Lyr, W, B, bs = wl.n_seqs, wl.n_layers, wl.window, wl.protect, wl.block_size
    rng = np.random.default_rng(cfg)
    samples = sorted({(0, 0), (S - 1, Lyr - 1), (int(rng.integers(S)), int(rng.integers(Lyr)))})
    lens = ses.lens_h.numpy().astype(np.int64)
    table = ses.table_h
    snap = {}
    for b, l in samples:
        L = int(lens[b])
        f0 = (L - W) // bs
        tail = list(range(f0 * bs, L))
        snap[b, l] = dict(
            q=wl.q_window[b, l].double().cpu().numpy(),
            k=gather_rows(wl.pool, table[b], list(range(L - W, L)), l, 0, bs).double().cpu().numpy(),
            tail=[gather_rows(wl.pool, table[b], tail, l, kv, bs).cpu() for kv in range(2)])
    sums_before = block_checksums(wl.pool)
    pool = ses.compress()
    torch.cuda.synchronize()
    print(f"[case] config {cfg} compressed; checking {samples}", flush=True)

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

    scores = ses.scores.view(S, Lyr, wl.n_kv_heads, -1)
    cand = ses.cand.view(S, Lyr, wl.n_kv_heads, -1)
    kept = ses.retained.view(S, Lyr, wl.n_kv_heads, -1)
    verdicts = {}
    for b, l in samples:
        s = ko.window_scores(snap[b, l]["q"], snap[b, l]["k"], B, unidirectional=uni)
        assert_scores_close(scores[b, l].cpu().numpy(), s, what=f"scores of ({b},{l})")
        kb = kept[b, l].cpu().numpy()
        cb = cand[b, l].cpu().numpy()
        for h in range(wl.n_kv_heads):
            v = adjudicate(s[h], wl.top_k, wl.budget, kb[h], cb[h], chunks=chunks)
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
            for h in range(wl.n_kv_heads):
                idx = list(range(p)) + [p + int(j) for j in kb[h]] + list(range(p + W - B, p + W))
                want = old[idx, h]
                got = new_rows[kv][:, h]
                assert torch.equal(want.view(torch.int16) if want.dtype == torch.bfloat16 else want,
                                   got.view(torch.int16) if got.dtype == torch.bfloat16 else got)
    print(f"[case] config {cfg} verdicts {verdicts}", flush=True)


@pytest.fixture(autouse=True)
def _release_memory():
    yield
    import gc
    gc.collect()
    if torch.cuda.is_available():
        torch.cuda.empty_cache()
