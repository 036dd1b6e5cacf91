"""GPU test of the periodic-compression serving trace (Distill-Llama-8B shapes,
reduced: 16 sequences x 2 layers, 24 events).  At every event that compresses
something, the call is checked against the oracle on the exact bytes it read:
scores within 1e-3, kept sets exact or adjudicated near-ties, the compacted
rows byte-exact against the old cache, tables/lengths/free list against the
oracle's pool model, and the schedule against the oracle's."""

import numpy as np
import pytest
import torch

from oracle import kara_oracle as ko
from parity import adjudicate, assert_scores_close

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from decode_kv_cache_kara_amd import kara
    from decode_kv_cache_kara_amd.trace import ServingTrace, TraceConfig, simulate_schedule


def test_serving_trace_small():
    print("[case] serving trace small", flush=True)
    cfg = TraceConfig(n_seqs=16, n_layers=2, init_len=1100, max_events=24, seed=77)
    tr = ServingTrace(cfg)
    c = cfg
    U_per_seq = c.n_layers * c.n_kv_heads
    checked = 0
    verdicts = {}
    while not tr.done():
        lens_before = tr.phys.copy()
        wm_before = tr.watermark.copy()
        batch = tr.next_event()
        # schedule against the oracle's definition (selection draws are the trace's)
        sel = tr.last_selected
        assert batch == ko.schedule_step(tr.step, c.period, c.window, tr.phys.tolist(),
                                         tr.watermark.tolist(), sel.tolist())
        if not batch:
            continue
        q = tr.window_queries(batch)
        pool_before = tr.pool.cpu()
        free_before = tr.blocks.snapshot()
        nb = len(batch)
        outs = dict(scores=torch.empty((nb * U_per_seq, c.window - c.protect), device="cuda"),
                    cand=torch.empty((nb * U_per_seq, c.top_k), dtype=torch.int32, device="cuda"),
                    retained=torch.empty((nb * U_per_seq, c.budget), dtype=torch.int32, device="cuda"))
        table_h, lens_h, new_table_h, new_lens_h = tr.compress(batch, q, outputs=outs)
        torch.cuda.synchronize()
        # bookkeeping against the oracle pool model
        fifo = ko.FifoPool(free_before)
        want_table, want_lens = ko.plan_compaction(table_h.numpy().astype(np.int64),
                                                   lens_h.numpy().astype(np.int64), c.window,
                                                   c.protect, c.budget, c.block_size, fifo)
        assert new_table_h.numpy().tolist() == want_table.tolist()
        assert new_lens_h.numpy().tolist() == want_lens.tolist()
        assert tr.blocks.snapshot() == fifo.ids()
        # scores and selections of every unit in the batch
        qn = q.cpu().double().numpy()
        pn = pool_before.double().numpy()
        S_ = outs["scores"].cpu().numpy().reshape(nb, c.n_layers, c.n_kv_heads, -1)
        cand = outs["cand"].cpu().numpy().reshape(nb, c.n_layers, c.n_kv_heads, -1)
        kept = outs["retained"].cpu().numpy().reshape(nb, c.n_layers, c.n_kv_heads, -1)
        for i in range(nb):
            L = int(lens_h[i])
            for l in range(c.n_layers):
                kw = ko.window_keys(pn, table_h[i].numpy(), L, c.window, l, c.n_kv_heads, c.block_size)
                s = ko.window_scores(qn[i, l], kw, c.protect)
                assert_scores_close(S_[i, l], s)
                for h in range(c.n_kv_heads):
                    v = adjudicate(s[h], c.top_k, c.budget, kept[i, l, h], cand[i, l, h])
                    assert not v.startswith("fail"), (tr.events, i, l, h, v)
                    verdicts[v] = verdicts.get(v, 0) + 1
        # compacted rows against the old cache, bit for bit
        pool_after = tr.pool.cpu()
        old16 = pool_before.view(torch.int16)
        new16 = pool_after.view(torch.int16)
        bs = c.block_size
        for i in range(nb):
            L = int(lens_h[i])
            start = L - c.window
            f0 = start // bs
            p = start - f0 * bs
            for l in range(c.n_layers):
                for h in range(c.n_kv_heads):
                    toks = (list(range(f0 * bs, start)) + [start + int(j) for j in kept[i, l, h]]
                            + list(range(L - c.protect, L)))
                    for kv in range(2):
                        src = torch.stack([old16[l, kv, int(table_h[i, t // bs]), h, t % bs] for t in toks])
                        dst = torch.stack([new16[l, kv, int(new_table_h[i, (f0 * bs + n) // bs]), h, (f0 * bs + n) % bs]
                                           for n in range(len(toks))])
                        assert torch.equal(src, dst)
        checked += 1
    print("[case] events", tr.events, "checked", checked, verdicts, flush=True)
    assert checked >= 3
    # lengths follow the host replay of the schedule
    n_events, _, _ = simulate_schedule(cfg)
    assert tr.events == n_events
