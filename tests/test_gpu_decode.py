"""GPU parity of the decode-side entry points around the compression step:
kara_append (K/V into the paged cache, query states into the ring),
kara_compress_ring (window query states read from the ring) and
kara_decode_attention (attention over the paged, possibly compacted, cache),
each through the C ABI against the oracle; and a small decode loop that
appends, compresses on the periodic schedule and attends over the compacted
tables, checked against the oracle's logical sequences."""

import numpy as np
import pytest
import torch

from oracle import kara_oracle as ko
from parity import adjudicate, assert_scores_close, bits

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from decode_kv_cache_kara_amd import kara, runner, synth


def say(*a):
    print("[case]", *a, flush=True)


ATT_RTOL = 2e-4   # fp32 accumulation over <= 32k tokens against float64


def assert_attention_close(got, want, what="attention"):
    got = np.asarray(got, dtype=np.float64)
    scale = np.abs(want).max(axis=-1, keepdims=True) + 1e-30
    err = np.abs(got - want) / scale
    assert err.max() <= ATT_RTOL, f"{what}: max error {err.max():.3e} of the row scale"
    return float(err.max())


def random_cache(seed, S, Lyr, Hkv, D, bs, lens, dtype, extra=7):
    g = torch.Generator().manual_seed(seed)
    nblk = [-(-L // bs) for L in lens]
    NB = sum(nblk) + extra
    MB = max(nblk) + 2
    perm = torch.randperm(NB, generator=g)
    table = torch.full((S, MB), -1, dtype=torch.int32)
    cur = 0
    for b in range(S):
        table[b, :nblk[b]] = perm[cur:cur + nblk[b]].to(torch.int32)
        cur += nblk[b]
    pool = torch.randn((Lyr, 2, NB, Hkv, bs, D), generator=g).to(dtype)
    return pool, table


ATT_CASES = {
    "bf16-d128-g4-ragged": dict(S=5, Lyr=2, Hq=32, Hkv=8, D=128, bs=16, lens=[1, 17, 255, 256, 1100],
                                dtype=torch.bfloat16, qs=0.3),
    "bf16-d128-g5-long": dict(S=2, Lyr=1, Hq=40, Hkv=8, D=128, bs=16, lens=[4097, 3000], dtype=torch.bfloat16,
                              qs=0.2),
    "bf16-d64-g3": dict(S=3, Lyr=1, Hq=6, Hkv=2, D=64, bs=8, lens=[9, 300, 77], dtype=torch.bfloat16, qs=0.5),
    "bf16-d128-g8-sharp": dict(S=2, Lyr=1, Hq=16, Hkv=2, D=128, bs=16, lens=[500, 33], dtype=torch.bfloat16,
                               qs=1.5),
    "fp32-d64-g2": dict(S=2, Lyr=1, Hq=4, Hkv=2, D=64, bs=16, lens=[256, 40], dtype=torch.float32, qs=1.0),
    "fp32-d128-g1": dict(S=2, Lyr=1, Hq=2, Hkv=2, D=128, bs=4, lens=[3, 600], dtype=torch.float32, qs=1.0),
}


def run_attention_case(name, c, cache_seed=11, q_seed=12):
    pool, table = random_cache(cache_seed, c["S"], c["Lyr"], c["Hkv"], c["D"], c["bs"], c["lens"], c["dtype"])
    g = torch.Generator().manual_seed(q_seed)
    q = (torch.randn((c["S"], c["Hq"], c["D"]), generator=g) * c["qs"]).to(c["dtype"])
    shape = kara.kara_shape(c["Lyr"], c["Hq"], c["Hkv"], c["D"], c["bs"], kara.dtype_code(c["dtype"]))
    lens_h = torch.tensor(c["lens"], dtype=torch.int32)
    ws = torch.empty(kara.kara_attention_workspace_bytes(shape, c["S"], max(c["lens"])), dtype=torch.uint8,
                     device="cuda")
    pd, td, qd = pool.cuda(), table.cuda(), q.cuda()
    pn = pool.double().numpy()
    worst = 0.0
    for layer in range(c["Lyr"]):
        out = torch.full((c["S"], c["Hq"], c["D"]), float("nan"), device="cuda")
        kara.kara_decode_attention(shape, layer, qd, pd, td, lens_h, lens_h.cuda(), out, ws)
        torch.cuda.synchronize()
        got = out.cpu().numpy()
        for b in range(c["S"]):
            want = ko.decode_attention(q[b].double().numpy(), pn, table[b].numpy(), c["lens"][b], layer, c["bs"])
            worst = max(worst, assert_attention_close(got[b], want, f"{name} seq {b} layer {layer}"))
    return worst


@pytest.mark.parametrize("name", list(ATT_CASES))
def test_decode_attention(name):
    say("decode attention", name)
    worst = run_attention_case(name, ATT_CASES[name])
    say(name, "max error", worst)


def random_attention_case(seed):
    """A seeded decode-attention shape: 1-6 sequences, 1-2 layers, G = 1 … 8,
    1-4 KV heads, head size 64 or 128, block size 4, 8 or 16, bf16 or float32,
    lengths from 1 to 5000 with some placed at the 512- and 1024-token split
    boundaries."""
    rng = np.random.default_rng(9500 + seed)
    S = int(rng.integers(1, 7))
    Hkv = int(rng.integers(1, 5))
    G = int(rng.integers(1, 9))
    edges = [1, 511, 512, 513, 1023, 1024, 1025, 2048, 2049]
    lens = [int(rng.choice(edges)) if rng.random() < 0.4 else int(rng.integers(1, 5001)) for _ in range(S)]
    return dict(S=S, Lyr=int(rng.integers(1, 3)), Hq=G * Hkv, Hkv=Hkv, D=int(rng.choice([64, 128])),
                bs=int(rng.choice([4, 8, 16])), lens=lens,
                dtype=torch.bfloat16 if rng.random() < 0.7 else torch.float32,
                qs=float(rng.choice([0.1, 0.5, 1.5])))


@pytest.mark.parametrize("seed", range(12))
def test_decode_attention_random_shapes(seed):
    c = random_attention_case(seed)
    say("decode attention, random shape", seed, {k: str(v) for k, v in c.items()})
    worst = run_attention_case(f"random {seed}", c, cache_seed=100 + seed, q_seed=200 + seed)
    say(seed, "max error", worst)


def test_decode_attention_large_launch_1024_token_splits():
    """A launch with enough work for 1024-token splits (512 sequences of
    1025-1100 tokens, 8 KV heads: at least 8192 workgroups of 1024 tokens),
    Qwen3-14B-shaped heads (G = 5, D = 128); sampled sequences, including both
    ends of the batch, against the oracle on their own blocks."""
    say("decode attention, 1024-token splits")
    S, Hq, Hkv, D, bs = 512, 40, 8, 128, 16
    rng = np.random.default_rng(21)
    lens = rng.integers(1025, 1101, S).astype(np.int32)
    nblk = (lens + bs - 1) // bs
    NB, MB = int(nblk.sum()), int(nblk.max())
    assert int(((lens + 1023) // 1024).sum()) * Hkv >= 8192
    perm = rng.permutation(NB).astype(np.int32)
    table = np.full((S, MB), -1, dtype=np.int32)
    off = np.concatenate([[0], np.cumsum(nblk)])
    for b in range(S):
        table[b, :nblk[b]] = perm[off[b]:off[b + 1]]
    g = torch.Generator(device="cuda").manual_seed(22)
    pool = torch.randn((1, 2, NB, Hkv, bs, D), generator=g, device="cuda").to(torch.bfloat16)
    q = (torch.randn((S, Hq, D), generator=g, device="cuda") * 0.3).to(torch.bfloat16)
    shape = kara.kara_shape(1, Hq, Hkv, D, bs, kara.KARA_BF16)
    lens_h = torch.from_numpy(lens)
    ws = torch.empty(kara.kara_attention_workspace_bytes(shape, S, int(lens.max())), dtype=torch.uint8,
                     device="cuda")
    out = torch.full((S, Hq, D), float("nan"), device="cuda")
    kara.kara_decode_attention(shape, 0, q, pool, torch.from_numpy(table).cuda(), lens_h, lens_h.cuda(), out, ws)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    worst = 0.0
    for b in [0, 1, 2, 100, 255, 256, 400, 509, 510, 511]:
        blocks = torch.from_numpy(table[b, :nblk[b]].astype(np.int64)).cuda()
        sub = pool.index_select(2, blocks).cpu().double().numpy()
        want = ko.decode_attention(q[b].cpu().double().numpy(), sub, np.arange(nblk[b], dtype=np.int32),
                                   int(lens[b]), 0, bs)
        worst = max(worst, assert_attention_close(got[b], want, f"1024-token splits seq {b}"))
    say("1024-token splits max error", worst)


def test_decode_attention_validates():
    shape = kara.kara_shape(1, 18, 2, 128, 16, kara.KARA_BF16)     # G = 9
    lens = torch.tensor([5], dtype=torch.int32)
    dummy = torch.empty(16, dtype=torch.uint8, device="cuda")
    with pytest.raises(kara.KaraError):
        kara.kara_decode_attention(shape, 0, dummy, torch.empty((1, 2, 1, 2, 16, 128), dtype=torch.bfloat16,
                                   device="cuda"), torch.zeros((1, 1), dtype=torch.int32, device="cuda"),
                                   lens, lens.cuda(), torch.empty((1, 18, 128), device="cuda"), dummy)
    shape = kara.kara_shape(1, 4, 2, 128, 16, kara.KARA_BF16)
    with pytest.raises(kara.KaraError):          # length beyond the table
        kara.kara_decode_attention(shape, 0, dummy, torch.empty((1, 2, 1, 2, 16, 128), dtype=torch.bfloat16,
                                   device="cuda"), torch.zeros((1, 1), dtype=torch.int32, device="cuda"),
                                   torch.tensor([17], dtype=torch.int32), lens.cuda(),
                                   torch.empty((1, 4, 128), device="cuda"), dummy)


@pytest.mark.parametrize("layer", [-1, 1])
def test_append_writes_cache_rows_and_ring(layer):
    say("append layer", layer)
    S, Lyr, Hq, Hkv, D, bs, W, n_slots = 3, 2, 8, 2, 128, 16, 64, 5
    dtype = torch.bfloat16
    pool, table = random_cache(21, S, Lyr, Hkv, D, bs, [40, 17, 70], dtype)
    shape = kara.kara_shape(Lyr, Hq, Hkv, D, bs, kara.KARA_BF16)
    g = torch.Generator().manual_seed(22)
    n_l = Lyr if layer < 0 else 1
    q = torch.randn((S, n_l, Hq, D), generator=g).to(dtype)
    k = torch.randn((S, n_l, Hkv, D), generator=g).to(dtype)
    v = torch.randn((S, n_l, Hkv, D), generator=g).to(dtype)
    positions = torch.tensor([39, 16, 5], dtype=torch.int32)      # 16: first row of a new block
    slots = torch.tensor([4, 0, 2], dtype=torch.int32)
    counts = torch.tensor([1000, 63, 64], dtype=torch.int32)      # ring positions 40, 63, 0
    ring = torch.randn((n_slots, Lyr, W, Hq, D), generator=g).to(dtype)
    before_pool, before_ring = pool.clone(), ring.clone()
    pd, rd = pool.cuda(), ring.cuda()
    qr = kara.QueryRing(rd, slots.cuda(), counts.cuda())
    if layer < 0:
        kara.kara_append(shape, W, -1, q.cuda(), k.cuda(), v.cuda(), pd, table.cuda(), positions.cuda(), qr)
    else:
        kara.kara_append(shape, W, layer, q[:, 0].contiguous().cuda(), k[:, 0].contiguous().cuda(),
                         v[:, 0].contiguous().cuda(), pd, table.cuda(), positions.cuda(), qr)
    torch.cuda.synchronize()
    want_pool, want_ring = before_pool.clone(), before_ring.clone()
    layers = range(Lyr) if layer < 0 else [layer]
    for b in range(S):
        t = int(positions[b])
        for i, l in enumerate(layers):
            want_pool[l, 0, table[b, t // bs], :, t % bs] = k[b, i]
            want_pool[l, 1, table[b, t // bs], :, t % bs] = v[b, i]
            want_ring[slots[b], l, int(counts[b]) % W] = q[b, i]
    assert torch.equal(bits(pd.cpu()), bits(want_pool))
    assert torch.equal(bits(rd.cpu()), bits(want_ring))


@pytest.mark.parametrize("cfg", [0, 1, 3])
def test_compress_ring_equals_compress(cfg):
    """The same windows, once as an array and once scattered into a ring with
    arbitrary slots and token counts, give bit-identical results (cfg 3's
    shape: the two-key-block scorer)."""
    say("compress ring", cfg)
    over = {1: dict(n_seqs=3, n_layers=2, lens=(1100, 3000)),
            3: dict(n_seqs=2, n_layers=2, lens=(2100, 4000))}.get(cfg, {})
    wl = synth.make_workload(cfg, device="cuda", **over)
    S, Lyr, W = wl.n_seqs, wl.n_layers, wl.window
    n_slots = S + 3
    slots = torch.randperm(n_slots, generator=torch.Generator().manual_seed(5))[:S].to(torch.int32)
    counts = torch.tensor([W + 17 + 1000 * b for b in range(S)], dtype=torch.int32)
    ring = torch.zeros((n_slots, Lyr, W) + wl.q_window.shape[3:], dtype=wl.dtype, device="cuda")
    for b in range(S):
        n = int(counts[b])
        idx = torch.tensor([(n - W + i) % W for i in range(W)], device="cuda")
        ring[int(slots[b]), :, idx] = wl.q_window[b]
    pool0 = wl.pool.clone()
    a = runner.Session(wl)
    pa = a.compress()
    torch.cuda.synchronize()
    pool_a = wl.pool.clone()
    wl.pool.copy_(pool0)
    b_ = runner.Session(wl)
    pb = b_.new_pool()
    qr = kara.QueryRing(ring, slots.cuda(), counts.cuda())
    kara.kara_compress_ring(b_.shape, b_.params, qr, wl.pool, b_.table_h, b_.table_d, b_.lens_h, b_.lens_d, pb,
                            b_.new_table_h, b_.new_table_d, b_.new_lens_h, b_.workspace,
                            scores_out=b_.scores, cand_out=b_.cand, retained_out=b_.retained)
    torch.cuda.synchronize()
    assert torch.equal(bits(a.scores), bits(b_.scores))
    assert torch.equal(a.cand, b_.cand) and torch.equal(a.retained, b_.retained)
    assert torch.equal(bits(pool_a), bits(wl.pool))
    assert torch.equal(a.new_table_h, b_.new_table_h) and pa.snapshot() == pb.snapshot()


def test_decode_loop_append_compress_attend():
    """Sequences decode token by token: every step appends K/V and query
    states; every P steps the schedule picks sequences whose window holds
    only new tokens, they are compressed from the ring, and decode attention
    over the compacted tables is compared with the oracle's attention over
    the logical sequences (prefix, kept tokens, protected tokens, new ones)."""
    say("decode loop")
    S, Lyr, Hq, Hkv, D, bs = 4, 2, 8, 2, 128, 16
    W, B, K, R, P = 128, 16, 8, 24, 40
    dtype = torch.bfloat16
    g = torch.Generator().manual_seed(31)
    init = [150, 200, 129, 260]
    MB = 64
    NB = S * MB
    shape = kara.kara_shape(Lyr, Hq, Hkv, D, bs, kara.KARA_BF16)
    params = kara.kara_params(W, B, K, R, 0)
    pool = torch.zeros((Lyr, 2, NB, Hkv, bs, D), dtype=dtype, device="cuda")
    blocks = kara.Pool(NB, list(range(NB)))
    table = torch.full((S, MB), -1, dtype=torch.int32)
    ring = torch.zeros((S, Lyr, W, Hq, D), dtype=dtype, device="cuda")
    slots_d = torch.arange(S, dtype=torch.int32, device="cuda")
    # host model: per sequence the logical rows [Lyr, 2, Hkv, D] of the cache, and the query history
    logical = [[] for _ in range(S)]
    history = [[] for _ in range(S)]
    phys = [0] * S
    produced = [0] * S
    watermark = [0] * S
    ws_c = torch.empty(max(kara.kara_workspace_bytes(shape, params, S), 256), dtype=torch.uint8, device="cuda")
    events = 0
    checked_units = 0

    def step_tokens(active):
        n = len(active)
        q = (torch.randn((n, Lyr, Hq, D), generator=g) * 0.3).to(dtype)
        k = (torch.randn((n, Lyr, Hkv, D), generator=g) * 0.3).to(dtype)
        v = torch.randn((n, Lyr, Hkv, D), generator=g).to(dtype)
        for i, b in enumerate(active):
            if phys[b] % bs == 0:
                table[b, phys[b] // bs] = blocks.alloc(1)[0]
        pos = torch.tensor([phys[b] for b in active], dtype=torch.int32, device="cuda")
        cnt = torch.tensor([produced[b] for b in active], dtype=torch.int32, device="cuda")
        sl = torch.tensor(active, dtype=torch.int32, device="cuda")
        qr = kara.QueryRing(ring, sl, cnt)
        kara.kara_append(shape, W, -1, q.cuda(), k.cuda(), v.cuda(), pool, table[active].cuda().contiguous(),
                         pos, qr)
        for i, b in enumerate(active):
            logical[b].append(torch.stack([k[i], v[i]], dim=1))   # [Lyr, 2, Hkv, D]
            history[b].append(q[i].float().numpy())
            phys[b] += 1
            produced[b] += 1

    for t in range(max(init)):
        step_tokens([b for b in range(S) if phys[b] < init[b]])
    torch.cuda.synchronize()
    for step in range(1, 4 * P + 1):
        step_tokens(list(range(S)))
        sel = torch.ones(S, dtype=torch.uint8)
        batch = kara.kara_schedule_step(step, P, W, torch.tensor(phys, dtype=torch.int32),
                                        torch.tensor(watermark, dtype=torch.int32), sel)
        if not batch:
            continue
        torch.cuda.synchronize()
        nb = len(batch)
        lens_h = torch.tensor([phys[b] for b in batch], dtype=torch.int32)
        tab_h = table[batch].contiguous()
        new_tab_h, new_lens_h = torch.empty_like(tab_h), torch.empty_like(lens_h)
        new_tab_d = torch.empty_like(tab_h).cuda()
        cnt = torch.tensor([produced[b] for b in batch], dtype=torch.int32, device="cuda")
        qr = kara.QueryRing(ring, torch.tensor(batch, dtype=torch.int32, device="cuda"), cnt)
        U = nb * Lyr * Hkv
        scores = torch.empty((U, W - B), device="cuda")
        kept = torch.empty((U, R), dtype=torch.int32, device="cuda")
        candd = torch.empty((U, K), dtype=torch.int32, device="cuda")
        kara.kara_compress_ring(shape, params, qr, pool, tab_h, tab_h.cuda(), lens_h, lens_h.cuda(), blocks,
                                new_tab_h, new_tab_d, new_lens_h, ws_c, scores_out=scores, cand_out=candd,
                                retained_out=kept)
        torch.cuda.synchronize()
        events += 1
        sc = scores.cpu().numpy().reshape(nb, Lyr, Hkv, -1)
        kp = kept.cpu().numpy().reshape(nb, Lyr, Hkv, R)
        cd = candd.cpu().numpy().reshape(nb, Lyr, Hkv, K)
        for i, b in enumerate(batch):
            L = phys[b]
            # scores from the oracle on the window's query history and logical keys
            qwin = ko.window_queries(history[b], W)                      # [Lyr, W, Hq, D]
            for l in range(Lyr):
                kwin = torch.stack([logical[b][t][l, 0] for t in range(L - W, L)]).double().numpy()
                s = ko.window_scores(qwin[l], kwin, B)
                assert_scores_close(sc[i, l], s)
                for h in range(Hkv):
                    v_ = adjudicate(s[h], K, R, kp[i, l, h], cd[i, l, h])
                    assert not v_.startswith("fail"), (step, b, l, h, v_)
                    checked_units += 1
            # the logical sequence after compaction (per layer and head the kept set differs)
            start = L - W
            newrows = []
            for n in range(start):
                newrows.append(logical[b][n])
            for r in range(R):
                row = torch.empty_like(logical[b][0])
                for l in range(Lyr):
                    for h in range(Hkv):
                        row[l, :, h] = logical[b][start + int(kp[i, l, h, r])][l, :, h]
                newrows.append(row)
            newrows += logical[b][L - B:L]
            logical[b] = newrows
            phys[b] = int(new_lens_h[i])
            assert phys[b] == len(logical[b])
            table[b] = new_tab_h[i]
            watermark[b] = phys[b] - B
        # decode attention over every sequence's current (compacted) cache
        qd = (torch.randn((S, Hq, D), generator=g) * 0.3).to(dtype)
        lens_all = torch.tensor(phys, dtype=torch.int32)
        ws = torch.empty(kara.kara_attention_workspace_bytes(shape, S, max(phys)), dtype=torch.uint8,
                         device="cuda")
        for l in range(Lyr):
            out = torch.empty((S, Hq, D), device="cuda")
            kara.kara_decode_attention(shape, l, qd.cuda(), pool, table.cuda(), lens_all, lens_all.cuda(), out, ws)
            torch.cuda.synchronize()
            got = out.cpu().numpy()
            for b in range(S):
                kk = torch.stack([r[l, 0] for r in logical[b]]).double().numpy()    # [L, Hkv, D]
                vv = torch.stack([r[l, 1] for r in logical[b]]).double().numpy()
                nbk = -(-len(logical[b]) // bs)
                flat = np.zeros((1, 2, nbk, Hkv, bs, D))
                for tkn in range(len(logical[b])):
                    flat[0, 0, tkn // bs, :, tkn % bs] = kk[tkn]
                    flat[0, 1, tkn // bs, :, tkn % bs] = vv[tkn]
                want = ko.decode_attention(qd[b].double().numpy(), flat, np.arange(nbk), len(logical[b]), 0, bs)
                assert_attention_close(got[b], want, f"step {step} seq {b} layer {l}")
    say("decode loop events", events, "units checked", checked_units)
    assert events >= 2 and checked_units > 0


@pytest.fixture(autouse=True)
def _release_memory():
    yield
    import gc
    gc.collect()
    if torch.cuda.is_available():
        torch.cuda.empty_cache()
