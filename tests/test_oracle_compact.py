"""Pins of the oracle's paged-cache bookkeeping and compaction: the worked
block example, a tag test (every row records where it came from), pool
conservation, FIFO order, and the KV-size arithmetic of the pages."""

import json
import math
import os

import numpy as np
import pytest

from oracle import kara_oracle as ko

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def tagged_pool(Lyr, NB, Hkv, bs, D):
    """Rows whose first four entries record (layer, K/V, block, head, slot)."""
    pool = np.zeros((Lyr, 2, NB, Hkv, bs, D), dtype=np.int64)
    for l in range(Lyr):
        for kv in range(2):
            for blk in range(NB):
                for h in range(Hkv):
                    for o in range(bs):
                        pool[l, kv, blk, h, o, :4] = (l * 2 + kv, blk, h, o)
    return pool


def tag_of_token(table_row, t, bs, l, kv, h):
    return (l * 2 + kv, int(table_row[t // bs]), h, t % bs)


def make_case(seed, S=3, Lyr=2, Hkv=2, bs=4, D=5, W=12, B=3, R=4, extra=6):
    rng = np.random.default_rng(seed)
    lens = rng.integers(W, W + 15, size=S)
    nblk = [math.ceil(L / bs) for L in lens]
    need_fresh = sum(math.ceil(((L - W) % bs + R + B) / bs) for L in lens)
    NB = sum(nblk) + need_fresh + extra
    perm = rng.permutation(NB)
    MB = max(nblk)
    table = np.full((S, MB), -1, dtype=np.int64)
    cur = 0
    for b in range(S):
        table[b, :nblk[b]] = perm[cur:cur + nblk[b]]
        cur += nblk[b]
    free = perm[cur:].tolist()
    C = W - B
    retained = np.zeros((S, Lyr, Hkv, R), dtype=np.int64)
    for b in range(S):
        for l in range(Lyr):
            for h in range(Hkv):
                retained[b, l, h] = np.sort(rng.permutation(C)[:R])
    return dict(lens=lens, table=table, free=free, retained=retained, NB=NB, S=S, Lyr=Lyr,
                Hkv=Hkv, bs=bs, D=D, W=W, B=B, R=R)


def test_worked_block_example():
    with open(os.path.join(GOLD, "compaction_worked.json")) as f:
        w = json.load(f)
    L, W, B, R, bs = w["len"], w["window"], w["protect"], w["budget"], w["block_size"]
    table = np.arange(100, 100 + math.ceil(L / bs))[None, :]
    pool = ko.FifoPool([1, 2, 3, 4, 5])
    new_table, new_lens = ko.plan_compaction(table, [L], W, B, R, bs, pool)
    k = w["kept_positions"]
    assert new_table[0, :k].tolist() == table[0, :k].tolist()
    assert new_table[0, w["fresh_positions"]].tolist() == [1, 2]
    assert np.all(new_table[0, max(w["fresh_positions"]) + 1:] == -1)
    assert int(new_lens[0]) == w["new_len"]
    assert pool.ids() == [3, 4, 5] + table[0, w["freed_positions"]].tolist()


@pytest.mark.parametrize("seed", range(8))
def test_tag_gather(seed):
    c = make_case(seed)
    pool_arr = tagged_pool(c["Lyr"], c["NB"], c["Hkv"], c["bs"], c["D"])
    fifo = ko.FifoPool(c["free"])
    new_table, new_lens = ko.plan_compaction(c["table"], c["lens"], c["W"], c["B"], c["R"], c["bs"], fifo)
    out = ko.apply_compaction(pool_arr, c["table"], c["lens"], new_table, c["W"], c["B"], c["R"],
                              c["bs"], c["retained"])
    bs = c["bs"]
    for b in range(c["S"]):
        L = int(c["lens"][b])
        Lnew = int(new_lens[b])
        assert Lnew == L - (c["W"] - c["B"]) + c["R"]
        start = L - c["W"]
        for l in range(c["Lyr"]):
            for h in range(c["Hkv"]):
                expect_tokens = (list(range(start))
                                 + [start + int(j) for j in c["retained"][b, l, h]]
                                 + list(range(L - c["B"], L)))
                assert len(expect_tokens) == Lnew
                for kv in range(2):
                    rows = ko.logical_tokens(out, new_table[b], Lnew, l, kv, h, bs)
                    got = [tuple(r[:4]) for r in rows]
                    want = [tag_of_token(c["table"][b], t, bs, l, kv, h) for t in expect_tokens]
                    assert got == want


@pytest.mark.parametrize("seed", range(8))
def test_pool_conservation_and_untouched_blocks(seed):
    c = make_case(seed)
    pool_arr = tagged_pool(c["Lyr"], c["NB"], c["Hkv"], c["bs"], c["D"])
    fifo = ko.FifoPool(c["free"])
    new_table, new_lens = ko.plan_compaction(c["table"], c["lens"], c["W"], c["B"], c["R"], c["bs"], fifo)
    out = ko.apply_compaction(pool_arr, c["table"], c["lens"], new_table, c["W"], c["B"], c["R"],
                              c["bs"], c["retained"])
    in_tables = [int(x) for row, L in zip(new_table, new_lens) for x in row[:math.ceil(int(L) / c["bs"])]]
    free_after = fifo.ids()
    assert len(in_tables) == len(set(in_tables))
    assert set(in_tables).isdisjoint(free_after)
    assert sorted(in_tables + free_after) == list(range(c["NB"]))
    fresh = set(in_tables) - {int(x) for x in c["table"].ravel() if x >= 0}
    # every block that is not fresh keeps its bytes
    for blk in range(c["NB"]):
        if blk not in fresh:
            assert np.array_equal(out[:, :, blk], pool_arr[:, :, blk])


def test_fifo_order():
    c = make_case(11)
    fifo = ko.FifoPool(c["free"])
    front = c["free"][:]
    new_table, _ = ko.plan_compaction(c["table"], c["lens"], c["W"], c["B"], c["R"], c["bs"], fifo)
    popped = []
    freed = []
    for b in range(c["S"]):
        L = int(c["lens"][b])
        f0 = (L - c["W"]) // c["bs"]
        n = math.ceil(((L - c["W"]) % c["bs"] + c["R"] + c["B"]) / c["bs"])
        popped += new_table[b, f0:f0 + n].tolist()
        freed += c["table"][b, f0:math.ceil(L / c["bs"])].tolist()
    assert popped == front[:len(popped)]
    assert fifo.ids() == front[len(popped):] + freed


def test_pool_exhaustion_changes_nothing():
    c = make_case(12)
    fifo = ko.FifoPool(c["free"][:3])
    with pytest.raises(ko.PoolExhausted):
        ko.plan_compaction(c["table"], c["lens"], c["W"], c["B"], c["R"], c["bs"], fifo)
    assert fifo.ids() == c["free"][:3]


def test_kv_bytes_of_the_pages():
    """The pages' 20 GB for 128K Qwen3-14B tokens in FP16, through the oracle's
    own cache layout: the bytes apply_compaction writes for one kept token of
    one layer (its K and V rows of every KV head) times tokens times layers."""
    with open(os.path.join(GOLD, "kv_bytes.json")) as f:
        w = json.load(f)
    Hkv, D, bs = w["n_kv_heads"], w["head_dim"], 16
    W, B = 32, 4
    L = W
    table = np.array([[0, 1]])
    pool = np.zeros((1, 2, 4, Hkv, bs, D), dtype=np.float16)
    pool[:, :, :2] = 1.0                                   # old blocks 0, 1; fresh blocks 2, 3 are empty
    new_table = np.array([[2, 3]])
    R = W - B                                              # keep every token of the region
    kept = np.arange(R).reshape(1, 1, 1, R).repeat(Hkv, axis=2)
    out = ko.apply_compaction(pool, table, np.array([L]), new_table, W, B, R, bs, kept)
    written = int((out[:, :, 2:] != pool[:, :, 2:]).sum()) * pool.itemsize
    per_token_per_layer = written // (R + B)
    assert per_token_per_layer == 2 * Hkv * D * w["elt_bytes"]
    assert w["tokens"] * w["n_layers"] * per_token_per_layer == w["bytes"] == 20 * 2 ** 30


def test_schedule_worked_example_oracle():
    """The oracle's schedule on a hand-worked step (period 128, W = 1024):
    sequence 0 holds 3000 tokens past its watermark (eligible), sequence 1 only
    500, sequence 2 is shorter than the window, sequence 3 was not selected;
    off the period and at step 0 nothing is compressed."""
    lens, wm, sel = [3000, 5000, 900, 2048], [0, 4500, 0, 0], [1, 1, 1, 0]
    assert ko.schedule_step(256, 128, 1024, lens, wm, sel) == [0]
    assert ko.schedule_step(128, 128, 1024, lens, wm, sel) == [0]
    assert ko.schedule_step(200, 128, 1024, lens, wm, sel) == []
    assert ko.schedule_step(0, 128, 1024, lens, wm, sel) == []
    # exactly W tokens past the watermark is eligible, one fewer is not
    assert ko.schedule_step(128, 128, 1024, [2024, 2023], [1000, 1000], [1, 1]) == [0]


def test_end_to_end_tiny_consistent():
    """compress() on a tagged tiny cache: stages agree with their separate calls."""
    rng = np.random.default_rng(21)
    S, Lyr, Hq, Hkv, D, bs, W, B, K, R = 2, 2, 4, 2, 4, 4, 16, 3, 4, 6
    lens = np.array([21, 30])
    nblk = [math.ceil(L / bs) for L in lens]
    NB = sum(nblk) + 20
    perm = rng.permutation(NB)
    table = np.full((S, max(nblk)), -1)
    table[0, :nblk[0]] = perm[:nblk[0]]
    table[1, :nblk[1]] = perm[nblk[0]:nblk[0] + nblk[1]]
    free = perm[sum(nblk):].tolist()
    pool = rng.normal(size=(Lyr, 2, NB, Hkv, bs, D))
    q = rng.normal(size=(S, Lyr, W, Hq, D))
    out = ko.compress(q, pool, table, lens, W, B, K, R, bs, free)
    for b in range(S):
        for l in range(Lyr):
            kwin = ko.window_keys(pool, table[b], int(lens[b]), W, l, Hkv, bs)
            s = ko.window_scores(q[b, l], kwin, B)
            np.testing.assert_array_equal(out["scores"][b, l], s)
            for h in range(Hkv):
                assert out["retained"][b, l, h].tolist() == ko.select_retained(s[h], K, R).tolist()
    assert out["lens"].tolist() == [L - (W - B) + R for L in lens]


@pytest.mark.parametrize("seed", range(4))
def test_window_keys_tags(seed):
    """The window gather reads the K rows (index 0) of the trailing W tokens, in order."""
    c = make_case(seed)
    pool_arr = tagged_pool(c["Lyr"], c["NB"], c["Hkv"], c["bs"], c["D"])
    for b in range(c["S"]):
        L = int(c["lens"][b])
        for l in range(c["Lyr"]):
            kw = ko.window_keys(pool_arr, c["table"][b], L, c["W"], l, c["Hkv"], c["bs"])
            for i in range(c["W"]):
                for h in range(c["Hkv"]):
                    assert tuple(kw[i, h, :4]) == tag_of_token(c["table"][b], L - c["W"] + i, c["bs"], l, 0, h)
