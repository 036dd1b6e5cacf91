"""GPU parity of the two ablations (Technical Summary: Kara, Experimental
Results, Ablation Studies) through the C ABI: unidirectional window scoring
(KARA_UNIDIRECTIONAL) and Token2Chunk off (KARA_NO_CHUNKS).

Bars as for the method itself: scores within 1e-3 relative of the oracle's
float64 scores; the selection replayed by the oracle on the GPU's own float32
scores equals the GPU's candidates and kept sets bit for bit; end-to-end kept
sets exact or adjudicated near-ties; bookkeeping and cache bytes exact."""

import numpy as np
import pytest
import torch

from oracle import kara_oracle as ko
from parity import (adjudicate, assert_scores_close, bits, expected_rows, oracle_scores, replay_selection,
                    tail_rows, tally)

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from decode_kv_cache_kara_amd import kara, runner, synth


def say(*a):
    print("[case]", *a, flush=True)


def gpu_workload(cfg=None, **over):
    return synth.make_workload(cfg, device="cpu", **over).to("cuda")


# Shapes chosen so that row chunks end at different key tiles (a chunk's last
# position decides how many tiles it reads), chunks straddle positions (G = 5),
# windows are ragged against the 64-key tile, and the protected buffer is
# empty or not.
UNI_CASES = {
    "tiny-fp32": dict(cfg=0),
    "ragged-bf16-d128-2chunks": dict(n_seqs=3, n_layers=2, n_q_heads=8, n_kv_heads=2, head_dim=128,
                                     block_size=16, window=200, protect=13, top_k=12, budget=40,
                                     lens=(200, 700), dtype=torch.bfloat16, qk_std=0.25),
    "ragged-bf16-d64-g3": dict(n_seqs=2, n_layers=1, n_q_heads=6, n_kv_heads=2, head_dim=64, block_size=8,
                               window=130, protect=2, top_k=9, budget=30, lens=(130, 400),
                               dtype=torch.bfloat16, qk_std=0.5),
    "fp32-d128-g5-noprotect": dict(n_seqs=2, n_layers=1, n_q_heads=5, n_kv_heads=1, head_dim=128,
                                   block_size=16, window=33, protect=0, top_k=5, budget=10,
                                   lens=[33, 50], dtype=torch.float32, qk_std=0.3),
    "window-1": dict(n_seqs=2, n_layers=1, n_q_heads=2, n_kv_heads=2, head_dim=64, block_size=4,
                     window=1, protect=0, top_k=1, budget=1, lens=[1, 9], dtype=torch.bfloat16),
    "qwen3-4b-1layer": dict(cfg=1),
    "qwen3-14b-shape-1seq": dict(n_seqs=1, n_layers=1, n_q_heads=40, n_kv_heads=8, head_dim=128,
                                 block_size=16, window=2048, protect=256, top_k=128, retention=0.3,
                                 lens=[8195], dtype=torch.bfloat16, qk_std=128 ** -0.5),
    "sharp-logits-bf16": dict(n_seqs=2, n_layers=2, n_q_heads=16, n_kv_heads=4, head_dim=128,
                              block_size=16, window=300, protect=40, top_k=16, budget=60,
                              lens=(300, 900), dtype=torch.bfloat16, qk_std=0.6),
}


def _workload(name):
    p = dict(UNI_CASES[name])
    cfg = p.pop("cfg", None)
    return gpu_workload(cfg, **p)


@pytest.mark.parametrize("name", list(UNI_CASES))
def test_unidirectional_score_stage(name):
    say("unidirectional score stage", name)
    wl = _workload(name)
    ses = runner.Session(wl, flags=kara.UNIDIRECTIONAL)
    out = torch.full((wl.n_units, wl.region), float("nan"), device="cuda")
    ses.score(out)
    torch.cuda.synchronize()
    orc = oracle_scores(wl, unidirectional=True).reshape(wl.n_units, wl.region)
    worst = assert_scores_close(out.cpu().numpy(), orc)
    # the ablation really changes the scores (a window of one token aside)
    if wl.window > 1:
        bi = oracle_scores(wl).reshape(wl.n_units, wl.region)
        assert not np.allclose(orc, bi, rtol=1e-2)
    say(name, "max rel err", worst)


def check_flags_e2e(wl, flags, case=None):
    uni = bool(flags & kara.UNIDIRECTIONAL)
    chunks = not (flags & kara.NO_CHUNKS)
    orc = oracle_scores(wl, unidirectional=uni)
    ses = runner.Session(wl, flags=flags)
    before = wl.pool.cpu().clone()
    pool = ses.compress()
    torch.cuda.synchronize()
    U, C, K, R = wl.n_units, wl.region, wl.top_k, wl.budget
    gs = ses.scores.cpu().numpy()
    worst = assert_scores_close(gs, orc.reshape(U, C))
    cand = ses.cand.cpu().numpy()
    kept = ses.retained.cpu().numpy()
    # replay on the GPU's own float32 scores: bit-exact
    replayed = replay_selection(gs, cand, kept, K, R, chunks=chunks)
    verdicts = {}
    for u in range(U):
        v = adjudicate(orc.reshape(U, C)[u], K, R, kept[u], cand[u], chunks=chunks)
        assert not v.startswith("fail"), (u, v)
        verdicts[v] = verdicts.get(v, 0) + 1
    table = ses.table_h.numpy().astype(np.int64)
    lens = ses.lens_h.numpy().astype(np.int64)
    fifo = ko.FifoPool(wl.free_ids)
    new_table, new_lens = ko.plan_compaction(table, lens, wl.window, wl.protect, R, wl.block_size, fifo)
    assert ses.new_table_h.numpy().tolist() == new_table.tolist()
    assert ses.new_lens_h.numpy().tolist() == new_lens.tolist()
    assert pool.snapshot() == fifo.ids()
    after = bits(wl.pool.cpu())
    old = bits(before)
    bs = wl.block_size
    for b in range(wl.n_seqs):
        f0 = (int(lens[b]) - wl.window) // bs
        n = (int(lens[b]) - wl.window) % bs + R + wl.protect
        for l in range(wl.n_layers):
            for h in range(wl.n_kv_heads):
                u = (b * wl.n_layers + l) * wl.n_kv_heads + h
                for kv in range(2):
                    want = expected_rows(old, table, lens, wl.window, wl.protect, bs, kept[u], b, l, kv, h)
                    got = tail_rows(after, new_table, b, l, kv, h, f0, n, bs)
                    assert torch.equal(got, want), (b, l, h, kv)
    if case:
        tally(case, verdicts, worst, replayed)
    return verdicts


E2E_CASES = {
    "tiny-fp32": dict(cfg=0),
    "qwen3-4b-1layer": dict(cfg=1),
    "sharp-logits-bf16": UNI_CASES["sharp-logits-bf16"],
    "budget-below-k": dict(n_seqs=2, n_layers=1, n_q_heads=4, n_kv_heads=2, head_dim=128, block_size=16,
                           window=96, protect=16, top_k=20, budget=7, lens=(96, 200),
                           dtype=torch.bfloat16, qk_std=0.5),
    "budget-equals-k": dict(n_seqs=2, n_layers=1, n_q_heads=4, n_kv_heads=2, head_dim=64, block_size=8,
                            window=120, protect=8, top_k=15, budget=15, lens=(120, 300),
                            dtype=torch.bfloat16, qk_std=0.5),
}


@pytest.mark.parametrize("flags", [1, 2, 3])
@pytest.mark.parametrize("name", list(E2E_CASES))
def test_ablation_end_to_end(name, flags):
    say("ablation end to end", name, "flags", flags)
    p = dict(E2E_CASES[name])
    cfg = p.pop("cfg", None)
    wl = gpu_workload(cfg, **p)
    verdicts = check_flags_e2e(wl, flags, case=f"ablation {name} flags {flags}")
    say(name, flags, verdicts)


def random_ablation_case(seed):
    """A seeded shape and ablation: flags 1, 2 or 3; bf16 or float32, head size
    64 or 128, W = 1 … 1500, G = 1 … 8, random B, K and R (R below K too)."""
    rng = np.random.default_rng(9000 + seed)
    flags = int(rng.integers(1, 4))
    dtype = torch.bfloat16 if rng.random() < 0.7 else torch.float32
    D = 128 if rng.random() < 0.7 else 64
    W = int(rng.choice([int(rng.integers(1, 100)), int(rng.integers(100, 1501))]))
    G = int(rng.integers(1, 9))
    Hkv = int(rng.integers(1, 3))
    B = int(rng.integers(0, max(1, W // 4)))
    C = W - B
    K = int(rng.integers(1, C + 1))
    R = int(rng.integers(1, C + 1))
    return flags, dict(n_seqs=2, n_layers=1, n_q_heads=G * Hkv, n_kv_heads=Hkv, head_dim=D,
                       block_size=int(rng.choice([8, 16])), window=W, protect=B, top_k=K, budget=R,
                       lens=(W, W + int(rng.integers(0, 2000))), dtype=dtype,
                       qk_std=float(rng.choice([0.1, 0.3, 0.6])))


@pytest.mark.parametrize("seed", range(12))
def test_ablation_end_to_end_random_shapes(seed):
    flags, p = random_ablation_case(seed)
    say("ablation end to end, random shape", seed, "flags", flags,
        {k: str(p[k]) for k in ("window", "protect", "top_k", "budget", "n_q_heads", "n_kv_heads", "head_dim",
                                "dtype")})
    wl = synth.make_workload(None, seed=9000 + seed, device="cpu", **p).to("cuda")
    verdicts = check_flags_e2e(wl, flags, case=f"ablation random shapes flags {flags}")
    say(seed, flags, verdicts)


def test_no_chunks_differs_from_token2chunk():
    """On planted spans the Token2Chunk result and the top-R set differ."""
    say("no-chunks differs")
    wl = gpu_workload(1)
    a = runner.Session(wl)
    a.compress()
    base = wl.pool.clone()
    torch.cuda.synchronize()
    b = runner.Session(wl, flags=kara.NO_CHUNKS)
    b.compress()
    torch.cuda.synchronize()
    assert torch.equal(a.cand, b.cand)
    assert not torch.equal(a.retained, b.retained)
    del base


@pytest.fixture(autouse=True)
def _release_memory():
    yield
    import gc
    gc.collect()
    if torch.cuda.is_available():
        torch.cuda.empty_cache()
