"""GPU parity of the HIP path (through the C ABI) against the CPU oracle.

Inputs are seeded synthetic workloads; the oracle runs on the exact bytes the
kernels read.  Bars: window scores within 1e-3 relative; selection stages
bit-exact on the same float32 scores; compaction byte-exact; end-to-end
selections exact or, where the oracle's scores are near-equal, a valid result
under the adjudication rule of tests/parity.py.
"""

import math

import numpy as np
import pytest
import torch

from oracle import kara_oracle as ko
from parity import (SCORE_RTOL, adjudicate, assert_scores_close, bits, expected_rows, host_inputs,
                    oracle_scores, replay_selection, tail_rows, tally)

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from decode_kv_cache_kara_amd import kara, runner, synth


def say(*a):
    print("[case]", *a, flush=True)


def gpu_workload(cfg=None, seed=None, **over):
    wl = synth.make_workload(cfg, seed=seed, device="cpu", **over)
    return wl.to("cuda")


SCORE_CASES = {
    "tiny-fp32": dict(cfg=0),
    "ragged-bf16-d128": dict(n_seqs=3, n_layers=2, n_q_heads=8, n_kv_heads=2, head_dim=128, block_size=16,
                             window=200, protect=13, top_k=12, budget=40, lens=(200, 700),
                             dtype=torch.bfloat16, qk_std=0.25),
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
    # windows of up to 1024 keys held in registers: a ragged last wave (W = 1000,
    # region not a multiple of 16), the largest row count (G = 16), a tiny
    # window (two 16-key tiles per wave, most keys past the window), no
    # protected buffer
    "resident-w1000-g5": dict(n_seqs=2, n_layers=1, n_q_heads=10, n_kv_heads=2, head_dim=128, block_size=16,
                              window=1000, protect=123, top_k=40, budget=175, lens=(1000, 3000),
                              dtype=torch.bfloat16, qk_std=0.3),
    "resident-w1024-g16": dict(n_seqs=1, n_layers=1, n_q_heads=32, n_kv_heads=2, head_dim=128, block_size=16,
                               window=1024, protect=128, top_k=64, budget=179, lens=[5000],
                               dtype=torch.bfloat16, qk_std=0.2),
    "resident-w17-b0": dict(n_seqs=3, n_layers=2, n_q_heads=6, n_kv_heads=3, head_dim=128, block_size=8,
                            window=17, protect=0, top_k=3, budget=9, lens=(17, 90), dtype=torch.bfloat16,
                            qk_std=0.5),
    # windows over two key blocks (1024 + the rest): region inside the first
    # block (C = 900), region equal to the window (B = 0, C = 2048), a short
    # second block with G = 3
    "resident-w1500-c900": dict(n_seqs=2, n_layers=1, n_q_heads=8, n_kv_heads=2, head_dim=128, block_size=16,
                                window=1500, protect=600, top_k=50, budget=200, lens=(1500, 4000),
                                dtype=torch.bfloat16, qk_std=0.3),
    "resident-w2048-b0-g2": dict(n_seqs=1, n_layers=2, n_q_heads=4, n_kv_heads=2, head_dim=128, block_size=16,
                                 window=2048, protect=0, top_k=128, budget=600, lens=[2500],
                                 dtype=torch.bfloat16, qk_std=0.25),
    "resident-w1100-g3": dict(n_seqs=2, n_layers=1, n_q_heads=6, n_kv_heads=2, head_dim=128, block_size=16,
                              window=1100, protect=50, top_k=60, budget=300, lens=(1100, 3000),
                              dtype=torch.bfloat16, qk_std=0.4),
    # query rows move 32 per pair of tiles, i.e. 32 / G positions and 32 % G
    # heads: one head per position (G = 1), a carry on most pairs (G = 7, one
    # and two key blocks), and more heads than 32 (G = 40: no position step)
    "resident-w333-g1": dict(n_seqs=2, n_layers=1, n_q_heads=3, n_kv_heads=3, head_dim=128, block_size=16,
                             window=333, protect=33, top_k=20, budget=90, lens=(333, 1200),
                             dtype=torch.bfloat16, qk_std=0.4),
    "resident-w700-g7": dict(n_seqs=2, n_layers=1, n_q_heads=14, n_kv_heads=2, head_dim=128, block_size=16,
                             window=700, protect=60, top_k=30, budget=150, lens=(700, 2100),
                             dtype=torch.bfloat16, qk_std=0.3),
    "resident-w1300-g7": dict(n_seqs=1, n_layers=2, n_q_heads=7, n_kv_heads=1, head_dim=128, block_size=16,
                              window=1300, protect=100, top_k=50, budget=260, lens=[2900],
                              dtype=torch.bfloat16, qk_std=0.3),
    "resident-w40-g40": dict(n_seqs=2, n_layers=1, n_q_heads=40, n_kv_heads=1, head_dim=128, block_size=8,
                             window=40, protect=4, top_k=6, budget=14, lens=(40, 99),
                             dtype=torch.bfloat16, qk_std=0.4),
    # the largest unit the resident scorer takes: G * W = 16384 rows
    "resident-w2048-g8-max-rows": dict(n_seqs=1, n_layers=1, n_q_heads=8, n_kv_heads=1, head_dim=128,
                                       block_size=16, window=2048, protect=200, top_k=64, budget=500,
                                       lens=[2600], dtype=torch.bfloat16, qk_std=0.3),
}


def _case(name):
    p = dict(SCORE_CASES[name])
    cfg = p.pop("cfg", None)
    return gpu_workload(cfg, **p)


@pytest.mark.parametrize("name", list(SCORE_CASES))
def test_score_stage(name):
    say("score stage", name)
    wl = _case(name)
    ses = runner.Session(wl)
    out = torch.full((wl.n_units, wl.region), float("nan"), device="cuda")
    ses.score(out)
    torch.cuda.synchronize()
    orc = oracle_scores(wl).reshape(wl.n_units, wl.region)
    worst = assert_scores_close(out.cpu().numpy(), orc)
    say(name, "max rel err", worst)


@pytest.mark.parametrize("window,n_q_heads", [(256, 8), (1600, 8), (2048, 16)])
def test_score_stage_exact_fallback(window, n_q_heads):
    """One key made ~110 nats more attractive to one query than that query's
    first keys: with the first keys' maximum as the row's reference the sum
    would overflow float, so the workgroup must redo its row statistics with a
    running maximum.  The scores still match the oracle."""
    say("score stage exact fallback, window", window, "query heads", n_q_heads)
    wl = gpu_workload(None, n_seqs=2, n_layers=1, n_q_heads=n_q_heads, n_kv_heads=2, head_dim=128,
                      block_size=16, window=window, protect=32, top_k=8, budget=40,
                      lens=[window + 44, window + 444], dtype=torch.bfloat16, qk_std=0.1)
    b, i, j = 0, 150, 200                      # sequence, query position, key position (window-local)
    q = wl.q_window[b, 0, i, 0].float()        # query head 0 belongs to KV head 0
    s = 110.0 * math.sqrt(128) / float(q @ q)
    L = int(wl.lens[b])
    t = L - wl.window + j
    blk = int(wl.table[b, t // wl.block_size])
    wl.pool[0, 0, blk, 0, t % wl.block_size] = (q * s).to(torch.bfloat16)
    kq = wl.pool[0, 0, blk, 0, t % wl.block_size].float()
    assert float(q @ kq) / math.sqrt(128) > 100.0
    ses = runner.Session(wl)
    out = torch.full((wl.n_units, wl.region), float("nan"), device="cuda")
    ses.score(out)
    torch.cuda.synchronize()
    orc = oracle_scores(wl).reshape(wl.n_units, wl.region)
    assert_scores_close(out.cpu().numpy(), orc)
    assert orc[0, j] > 0.9                     # the planted key took that row's whole weight


@pytest.mark.parametrize("window", [256, 2048])
def test_score_stage_exact_rerun_for_very_negative_logits(window):
    """One query row whose logits with every window key are about -60 nats:
    without a reference its normaliser falls below float's comfortable range,
    so the scorer must take the exact route (every row's maximum as its
    reference).  The scores still match the oracle."""
    say("score stage exact rerun, very negative logits")
    wl = gpu_workload(None, n_seqs=1, n_layers=1, n_q_heads=4, n_kv_heads=1, head_dim=128, block_size=16,
                      window=window, protect=32, top_k=8, budget=40, lens=[window + 344], dtype=torch.bfloat16,
                      qk_std=0.1)
    L = int(wl.lens[0])
    toks = torch.arange(L - wl.window, L)
    blk = wl.table[0].long()[toks // wl.block_size]
    off = toks % wl.block_size
    u = torch.ones(128, device="cuda") / math.sqrt(128)
    k = wl.pool[0, 0, blk, 0, off].float() + 2.0 * u           # every window key shares direction u
    wl.pool[0, 0, blk, 0, off] = k.to(torch.bfloat16)
    q = -(60.0 * math.sqrt(128) / 2.0) * u                       # logits about -60 nats with every key
    wl.q_window[0, 0, 77, 1] = q.to(torch.bfloat16)
    kq = wl.pool[0, 0, blk, 0, off].float() @ wl.q_window[0, 0, 77, 1].float() / math.sqrt(128)
    assert float(kq.max()) < -50.0
    ses = runner.Session(wl)
    out = torch.full((wl.n_units, wl.region), float("nan"), device="cuda")
    ses.score(out)
    torch.cuda.synchronize()
    orc = oracle_scores(wl).reshape(wl.n_units, wl.region)
    assert_scores_close(out.cpu().numpy(), orc)


REGIONS = [1, 7, 56, 187, 896, 1792, 2048]


@pytest.mark.parametrize("kind", ["normal", "ties", "coarse", "flat", "spiky"])
@pytest.mark.parametrize("C", REGIONS)
def test_topk_stage(kind, C):
    say("topk stage", kind, C)
    n_units = 24
    s = synth.random_scores(n_units, C, seed=C * 7 + len(kind), kind=kind)
    rng = np.random.default_rng(C)
    for K in sorted({1, min(C, 8), min(C, 64), min(C, 128), C, int(rng.integers(1, C + 1))}):
        out = torch.full((n_units, K), -7, dtype=torch.int32, device="cuda")
        kara.kara_topk(s.cuda(), K, out)
        torch.cuda.synchronize()
        got = out.cpu().numpy()
        for u in range(n_units):
            want = ko.topk_candidates(s[u].numpy(), K)
            assert got[u].tolist() == want.tolist(), (kind, C, K, u)


@pytest.mark.parametrize("kind", ["normal", "ties", "coarse", "flat", "spiky"])
@pytest.mark.parametrize("C", REGIONS)
def test_token2chunk_stage(kind, C):
    say("token2chunk stage", kind, C)
    n_units = 16
    s = synth.random_scores(n_units, C, seed=C * 11 + len(kind), kind=kind)
    rng = np.random.default_rng(C + 1)
    combos = {(1, 1), (min(C, 8), C), (min(C, 64), min(C, 179)), (min(C, 128), min(C, 537)),
              (min(C, 16), min(C, 8))}
    for _ in range(3):
        K = int(rng.integers(1, C + 1))
        combos.add((K, int(rng.integers(1, C + 1))))
    for K, R in sorted(combos):
        cand = np.stack([ko.topk_candidates(s[u].numpy(), K) for u in range(n_units)]).astype(np.int32)
        out = torch.full((n_units, R), -7, dtype=torch.int32, device="cuda")
        kara.kara_token2chunk(s.cuda(), torch.from_numpy(cand).cuda(), R, out)
        torch.cuda.synchronize()
        got = out.cpu().numpy()
        for u in range(n_units):
            want = ko.token2chunk(s[u].numpy(), cand[u], R)
            assert got[u].tolist() == want.tolist(), (kind, C, K, R, u)


COMPACT_CASES = {
    "tiny-fp32": dict(cfg=0),
    "bf16-unaligned": dict(n_seqs=3, n_layers=2, n_q_heads=8, n_kv_heads=2, head_dim=128, block_size=16,
                           window=100, protect=9, top_k=8, budget=30, lens=(100, 500), dtype=torch.bfloat16),
    "bf16-d64-bs8": dict(n_seqs=4, n_layers=1, n_q_heads=4, n_kv_heads=4, head_dim=64, block_size=8,
                         window=64, protect=5, top_k=4, budget=59, lens=(64, 300), dtype=torch.bfloat16),
    "qwen3-4b-1layer": dict(cfg=1),
}


@pytest.mark.parametrize("name", list(COMPACT_CASES))
def test_compact_stage(name):
    say("compact stage", name)
    p = dict(COMPACT_CASES[name])
    cfg = p.pop("cfg", None)
    wl = gpu_workload(cfg, **p)
    ses = runner.Session(wl, outputs=False)
    ret = synth.random_retained(wl.n_units, wl.region, wl.budget, seed=5).cuda()
    before = wl.pool.cpu().clone()
    pool = ses.new_pool()
    kara.kara_paged_compact(ses.shape, ses.params, wl.pool, ses.table_h, ses.table_d, ses.lens_h,
                            ses.lens_d, ret, pool, ses.new_table_h, ses.new_table_d, ses.new_lens_h)
    torch.cuda.synchronize()
    # oracle bookkeeping and copy on the same inputs
    table = ses.table_h.numpy().astype(np.int64)
    lens = ses.lens_h.numpy().astype(np.int64)
    fifo = ko.FifoPool(wl.free_ids)
    new_table, new_lens = ko.plan_compaction(table, lens, wl.window, wl.protect, wl.budget, wl.block_size, fifo)
    assert ses.new_table_h.numpy().tolist() == new_table.tolist()
    assert ses.new_table_d.cpu().numpy().tolist() == new_table.tolist()
    assert ses.new_lens_h.numpy().tolist() == new_lens.tolist()
    assert pool.snapshot() == fifo.ids()
    retained = ret.cpu().numpy().reshape(wl.n_seqs, wl.n_layers, wl.n_kv_heads, wl.budget)
    want = ko.apply_compaction(bits(before).numpy(), table, lens, new_table, wl.window, wl.protect,
                               wl.budget, wl.block_size, retained)
    got = bits(wl.pool.cpu()).numpy()
    assert np.array_equal(got, want)


E2E_CASES = {
    "tiny-fp32": dict(cfg=0),
    "qwen3-4b-1layer": dict(cfg=1),
    "sharp-logits-bf16": SCORE_CASES["sharp-logits-bf16"],
    "ragged-bf16-d64-g3": SCORE_CASES["ragged-bf16-d64-g3"],
    "budget-below-k": dict(n_seqs=2, n_layers=1, n_q_heads=4, n_kv_heads=2, head_dim=128, block_size=16,
                           window=96, protect=16, top_k=20, budget=7, lens=(96, 200), dtype=torch.bfloat16,
                           qk_std=0.5),
    "resident-w1000-g5": SCORE_CASES["resident-w1000-g5"],
    "resident-w1500-c900": SCORE_CASES["resident-w1500-c900"],
    "resident-w2048-b0-g2": SCORE_CASES["resident-w2048-b0-g2"],
}


def run_e2e(wl):
    ses = runner.Session(wl)
    before = wl.pool.cpu().clone()
    pool = ses.compress()
    torch.cuda.synchronize()
    return ses, pool, before


def check_e2e(wl, ses, pool, before, orc_scores, case=None):
    U, C = wl.n_units, wl.region
    gs = ses.scores.cpu().numpy()
    worst = assert_scores_close(gs, orc_scores.reshape(U, C))
    cand = ses.cand.cpu().numpy()
    kept = ses.retained.cpu().numpy()
    # the selection stages replayed on the GPU's own float32 scores: bit for bit
    replayed = replay_selection(gs, cand, kept, wl.top_k, wl.budget)
    verdicts = {}
    for u in range(U):
        v = adjudicate(orc_scores.reshape(U, C)[u], wl.top_k, wl.budget, kept[u], cand[u])
        assert not v.startswith("fail"), (u, v)
        verdicts[v] = verdicts.get(v, 0) + 1
    # bookkeeping does not depend on the selection: exact against the oracle
    table = ses.table_h.numpy().astype(np.int64)
    lens = ses.lens_h.numpy().astype(np.int64)
    fifo = ko.FifoPool(wl.free_ids)
    new_table, new_lens = ko.plan_compaction(table, lens, wl.window, wl.protect, wl.budget, wl.block_size, fifo)
    assert ses.new_table_h.numpy().tolist() == new_table.tolist()
    assert ses.new_table_d.cpu().numpy().tolist() == new_table.tolist()
    assert ses.new_lens_h.numpy().tolist() == new_lens.tolist()
    assert pool.snapshot() == fifo.ids()
    # the compacted cache holds exactly the rows of the GPU's kept set, bit for bit
    after = bits(wl.pool.cpu())
    old = bits(before)
    bs = wl.block_size
    for b in range(wl.n_seqs):
        f0 = (int(lens[b]) - wl.window) // bs
        n = (int(lens[b]) - wl.window) % bs + wl.budget + wl.protect
        for l in range(wl.n_layers):
            for h in range(wl.n_kv_heads):
                u = (b * wl.n_layers + l) * wl.n_kv_heads + h
                for kv in range(2):
                    want = expected_rows(old, table, lens, wl.window, wl.protect, bs, kept[u], b, l, kv, h)
                    got = tail_rows(after, new_table, b, l, kv, h, f0, n, bs)
                    assert torch.equal(got, want), (b, l, h, kv)
    # every block that is not fresh keeps its bytes
    fresh = {int(x) for row in new_table for x in row if x >= 0} - {int(x) for x in table.ravel() if x >= 0}
    keep = [i for i in range(wl.n_blocks) if i not in fresh]
    assert torch.equal(after[:, :, keep], old[:, :, keep])
    if case:
        tally(case, verdicts, worst, replayed)
    return verdicts


@pytest.mark.parametrize("name", list(E2E_CASES))
def test_compress_end_to_end(name):
    say("compress end to end", name)
    p = dict(E2E_CASES[name])
    cfg = p.pop("cfg", None)
    wl = gpu_workload(cfg, **p)
    orc = oracle_scores(wl)
    ses, pool, before = run_e2e(wl)
    verdicts = check_e2e(wl, ses, pool, before, orc, case=f"e2e {name}")
    say(name, verdicts)
    if name in ("tiny-fp32", "sharp-logits-bf16"):
        assert verdicts.get("exact", 0) == wl.n_units   # well-separated scores: no ties to adjudicate


def random_resident_case(seed):
    """A seeded shape for the resident-key scorer (bf16, head size 128): W over
    1..2048 (one or two key blocks), G = 1..8 with G * W <= 16384 rows, one or
    two KV heads, a random protected tail, K and R anywhere in [1, C] with
    R >= K, ragged sequence lengths, and a random logit scale."""
    rng = np.random.default_rng(7000 + seed)
    W = int(rng.choice([int(rng.integers(1, 200)), int(rng.integers(200, 1025)), int(rng.integers(1025, 2049))]))
    G = int(rng.integers(1, 9))
    while G * W > 16384:
        G -= 1
    Hkv = int(rng.integers(1, 3))
    B = int(rng.integers(0, max(1, W // 4)))
    C = W - B
    K = int(rng.integers(1, C + 1))
    R = int(rng.integers(K, C + 1)) if C > K else C
    return dict(n_seqs=2, n_layers=1, n_q_heads=G * Hkv, n_kv_heads=Hkv, head_dim=128, block_size=16,
                window=W, protect=B, top_k=K, budget=R, lens=(W, W + int(rng.integers(0, 3000))),
                dtype=torch.bfloat16, qk_std=float(rng.choice([0.1, 0.3, 0.6])))


@pytest.mark.parametrize("seed", range(24))
def test_compress_end_to_end_random_resident_shapes(seed):
    p = random_resident_case(seed)
    say("compress end to end, random resident shape", seed, {k: p[k] for k in ("window", "protect", "top_k",
                                                                              "budget", "n_q_heads", "n_kv_heads")})
    wl = gpu_workload(None, seed=7000 + seed, **p)
    orc = oracle_scores(wl)
    ses, pool, before = run_e2e(wl)
    verdicts = check_e2e(wl, ses, pool, before, orc, case="e2e random resident shapes")
    say(seed, verdicts)


def random_twopass_case(seed):
    """A seeded shape for the two-pass scorer: float32 (head size 64 or 128),
    bf16 with head size 64, or bf16 / 128 with a window over 2048 keys."""
    rng = np.random.default_rng(8000 + seed)
    kind = int(rng.integers(0, 4))
    dtype = torch.float32 if kind <= 1 else torch.bfloat16
    D = 64 if kind in (0, 2) else 128
    W = int(rng.integers(2049, 4097)) if kind == 3 else int(rng.integers(1, 1200))
    G = int(rng.integers(1, 5 if kind == 3 else 9))
    Hkv = int(rng.integers(1, 3))
    B = int(rng.integers(0, max(1, W // 4)))
    C = min(W - B, 2048)
    B = W - C
    K = int(rng.integers(1, C + 1))
    R = int(rng.integers(K, C + 1)) if C > K else C
    return dict(n_seqs=2, n_layers=1, n_q_heads=G * Hkv, n_kv_heads=Hkv, head_dim=D,
                block_size=int(rng.choice([8, 16])), window=W, protect=B, top_k=K, budget=R,
                lens=(W, W + int(rng.integers(0, 3000))), dtype=dtype, qk_std=float(rng.choice([0.1, 0.3, 0.6])))


@pytest.mark.parametrize("seed", range(16))
def test_compress_end_to_end_random_twopass_shapes(seed):
    p = random_twopass_case(seed)
    say("compress end to end, random two-pass shape", seed, {k: str(p[k]) for k in (
        "window", "protect", "top_k", "budget", "n_q_heads", "n_kv_heads", "head_dim", "dtype")})
    wl = gpu_workload(None, seed=8000 + seed, **p)
    orc = oracle_scores(wl)
    ses, pool, before = run_e2e(wl)
    verdicts = check_e2e(wl, ses, pool, before, orc, case="e2e random two-pass shapes")
    say(seed, verdicts)


def test_compress_matches_oracle_end_to_end_exactly_when_sets_agree():
    """Where the oracle's selection is reproduced, the whole step (cache bytes,
    tables, lengths, free list) equals the oracle's compress() output."""
    say("compress exact vs oracle compress()")
    wl = gpu_workload(0)
    q, pool_np, table, lens = host_inputs(wl)
    ses, pool, before = run_e2e(wl)
    kept = ses.retained.cpu().numpy().reshape(wl.n_seqs, wl.n_layers, wl.n_kv_heads, wl.budget)
    orc = ko.compress(q, pool_np, table, lens, wl.window, wl.protect, wl.top_k, wl.budget, wl.block_size,
                      wl.free_ids)
    assert np.array_equal(kept, orc["retained"])
    assert ses.new_table_h.numpy().tolist() == orc["table"].tolist()
    assert ses.new_lens_h.numpy().tolist() == orc["lens"].tolist()
    assert pool.snapshot() == orc["free_ids"]
    want = ko.apply_compaction(bits(before).numpy(), table, lens, orc["table"], wl.window, wl.protect,
                               wl.budget, wl.block_size, orc["retained"])
    assert np.array_equal(bits(wl.pool.cpu()).numpy(), want)


def test_compress_subset_leaves_other_sequences_untouched():
    say("compress subset")
    wl = gpu_workload(None, n_seqs=4, n_layers=2, n_q_heads=8, n_kv_heads=2, head_dim=128, block_size=16,
                      window=128, protect=16, top_k=8, budget=24, lens=(128, 600), dtype=torch.bfloat16)
    sel = [2, 0]
    sub = synth.Workload(**{**wl.__dict__})
    sub.n_seqs = len(sel)
    sub.q_window = wl.q_window[sel].contiguous()
    sub.table = wl.table[sel].contiguous()
    sub.lens = wl.lens[sel].contiguous()
    used_other = {int(x) for b in (1, 3) for x in wl.table[b].cpu().tolist() if x >= 0}
    before = wl.pool.cpu().clone()
    ses = runner.Session(sub)
    ses.compress()
    torch.cuda.synchronize()
    after = wl.pool.cpu()
    idx = sorted(used_other)
    assert torch.equal(bits(after[:, :, idx]), bits(before[:, :, idx]))


def test_determinism():
    say("determinism")
    wl = gpu_workload(1)
    ses = runner.Session(wl)
    before = wl.pool.clone()
    ses.compress()
    torch.cuda.synchronize()
    s1, c1, r1, p1 = ses.scores.clone(), ses.cand.clone(), ses.retained.clone(), wl.pool.clone()
    wl.pool.copy_(before)
    ses.compress()
    torch.cuda.synchronize()
    assert torch.equal(bits(ses.scores), bits(s1))
    assert torch.equal(ses.cand, c1) and torch.equal(ses.retained, r1)
    assert torch.equal(bits(wl.pool), bits(p1))


def test_errors_leave_state_unchanged_on_gpu():
    say("error path on gpu")
    wl = gpu_workload(0)
    ses = runner.Session(wl)
    pool = kara.Pool(wl.n_blocks, wl.free_ids[:1])     # too few fresh blocks
    before = wl.pool.clone()
    with pytest.raises(kara.KaraError) as e:
        ses.compress(pool=pool)
    assert e.value.status == kara.KARA_E_NOBLOCKS
    torch.cuda.synchronize()
    assert torch.equal(bits(wl.pool), bits(before))
    assert pool.snapshot() == wl.free_ids[:1]
