"""Host-side tests of libkara.so that need no GPU: every symbol of
include/kara.h is exported, the FIFO pool behaves as documented, and invalid
arguments are rejected before anything is touched (the device pointers passed
here are never valid, so any dereference would crash)."""

import ctypes
import os
import re

import pytest

from decode_kv_cache_kara_amd import kara

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = 0x10  # never dereferenced: validation fails first


def header_functions():
    with open(os.path.join(ROOT, "include", "kara.h")) as f:
        text = f.read()
    return sorted(set(re.findall(r"\b(kara_[a-z0-9_]+)\s*\(", text)))


def test_every_declared_symbol_is_exported():
    lib = ctypes.CDLL(kara.LIB_PATH)
    names = header_functions()
    assert len(names) >= 14
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(kara.EXPORTED)


def test_version():
    assert "gfx950" in kara.kara_version()


def test_pool_fifo():
    p = kara.Pool(10, [7, 3, 5, 1])
    assert p.num_free() == 4
    assert p.alloc(2) == [7, 3]
    p.free([9, 0])
    assert p.snapshot() == [5, 1, 9, 0]
    with pytest.raises(kara.KaraError) as e:
        p.alloc(5)
    assert e.value.status == kara.KARA_E_NOBLOCKS
    assert p.snapshot() == [5, 1, 9, 0]


@pytest.mark.parametrize("ids", [[1, 1], [5], [10], [-1]])
def test_pool_free_rejects(ids):
    p = kara.Pool(10, [5, 6])
    with pytest.raises(kara.KaraError) as e:
        p.free(ids)
    assert e.value.status == kara.KARA_E_INVAL
    assert p.snapshot() == [5, 6]


@pytest.mark.parametrize("n,ids", [(0, []), (4, [0, 0]), (4, [4]), (4, [-2])])
def test_pool_create_rejects(n, ids):
    with pytest.raises(kara.KaraError):
        kara.Pool(n, ids)


def shape(**kw):
    d = dict(n_layers=2, n_q_heads=8, n_kv_heads=2, head_dim=128, block_size=4, dtype=kara.KARA_BF16)
    d.update(kw)
    return kara.kara_shape(**d)


def params(**kw):
    d = dict(window=8, protect=2, top_k=2, budget=3)
    d.update(kw)
    return kara.kara_params(**d)


def test_workspace_bytes():
    sh, pr = shape(), params()
    n1 = kara.kara_workspace_bytes(sh, pr, 1)
    n4 = kara.kara_workspace_bytes(sh, pr, 4)
    assert 0 < n1 < n4
    assert kara.kara_workspace_bytes(sh, params(window=0), 1) == 0
    assert kara.kara_workspace_bytes(shape(head_dim=96), pr, 1) == 0
    # the ablation flags do not change the workspace
    for f in (kara.UNIDIRECTIONAL, kara.NO_CHUNKS, kara.UNIDIRECTIONAL | kara.NO_CHUNKS):
        assert kara.kara_workspace_bytes(sh, params(flags=f), 4) == n4
    assert kara.kara_workspace_bytes(sh, params(flags=8), 4) == 0


def _i32(vals):
    return (ctypes.c_int32 * len(vals))(*vals)


class Call:
    """A kara_compress call with valid host arguments and fake device pointers."""

    def __init__(self, **over):
        self.shape = over.pop("shape", shape())
        self.params = over.pop("params", params())
        self.lens = over.pop("lens", [10, 13])
        bs = self.shape.block_size
        self.max_blocks = over.pop("max_blocks", 5)
        self.n_blocks = over.pop("n_blocks", 20)
        table = over.pop("table", None)
        if table is None:
            table, nxt = [], 0
            for L in self.lens:
                n = -(-L // bs)
                row = list(range(nxt, nxt + n)) + [-1] * (self.max_blocks - n)
                nxt += n
                table += row
            free = list(range(nxt, self.n_blocks))
        else:
            free = over.pop("free")
        self.table = _i32(table)
        self.free = over.pop("free", free)
        self.pool = kara.Pool(self.n_blocks, self.free)
        self.new_table = _i32([0] * (len(self.lens) * self.max_blocks))
        self.new_lens = _i32([0] * len(self.lens))
        self.ws = over.pop("ws", kara.kara_workspace_bytes(self.shape, self.params, len(self.lens)))
        assert not over

    def run(self, q=FAKE * 16, kv=FAKE * 16):
        return kara.lib.kara_compress(
            ctypes.byref(self.shape), ctypes.byref(self.params), len(self.lens), q, kv,
            self.n_blocks, self.table, FAKE * 16, self.max_blocks, _i32(self.lens), FAKE * 16,
            self.pool.handle, self.new_table, FAKE * 16, self.new_lens, 256 * 16, self.ws, None,
            None, None, None, None)


@pytest.mark.parametrize("kw,status", [
    (dict(params=params(window=20)), kara.KARA_E_INVAL),            # L < W
    (dict(params=params(protect=8)), kara.KARA_E_INVAL),            # B >= W
    (dict(params=params(top_k=7)), kara.KARA_E_INVAL),              # K > C
    (dict(params=params(budget=0)), kara.KARA_E_INVAL),             # R < 1
    (dict(params=params(window=5000)), kara.KARA_E_INVAL),
    (dict(params=params(flags=4)), kara.KARA_E_INVAL),              # unknown ablation bit
    (dict(params=params(flags=-1)), kara.KARA_E_INVAL),
    (dict(shape=shape(head_dim=96)), kara.KARA_E_UNSUPPORTED),
    (dict(shape=shape(dtype=7)), kara.KARA_E_UNSUPPORTED),
    (dict(shape=shape(n_q_heads=7)), kara.KARA_E_INVAL),
    (dict(table=[0, 1, 2, -1, -1, 3, 4, 25, 5, -1], free=list(range(6, 20))), kara.KARA_E_INVAL),
    (dict(ws=0), kara.KARA_E_WORKSPACE),
    (dict(max_blocks=3), kara.KARA_E_INVAL),                        # length needs more blocks
])
def test_compress_rejects_before_side_effects(kw, status):
    c = Call(**kw)
    before = c.pool.snapshot()
    assert c.run() == status, kara.kara_last_error()
    assert kara.kara_last_error()
    assert c.pool.snapshot() == before
    assert list(c.new_lens) == [0, 0]


@pytest.mark.parametrize("arg", ["q", "kv"])
def test_compress_rejects_misaligned_state_arrays(arg):
    """The query states and the pool must be 16-byte aligned; an 8-byte offset
    is rejected before any side effect."""
    c = Call()
    before = c.pool.snapshot()
    assert c.run(**{arg: FAKE * 16 + 8}) == kara.KARA_E_INVAL
    assert "aligned" in kara.kara_last_error()
    assert c.pool.snapshot() == before
    assert list(c.new_lens) == [0, 0]


def test_compress_pool_exhaustion_changes_nothing():
    c = Call(n_blocks=8)   # 7 blocks used by the tables, 1 free, 2 x 2 fresh needed
    before = c.pool.snapshot()
    assert c.run() == kara.KARA_E_NOBLOCKS
    assert c.pool.snapshot() == before
    assert list(c.new_lens) == [0, 0]


def test_compress_rejects_duplicate_and_free_blocks():
    # block 2 appears in both tails
    c = Call(table=[0, 1, 2, -1, -1, 3, 4, 2, 5, -1], free=list(range(6, 20)))
    assert c.run() == kara.KARA_E_INVAL
    # block 4 is in sequence 1's tail and also listed free
    c = Call(table=[0, 1, 2, -1, -1, 3, 4, 6, 5, -1], free=[4] + list(range(7, 20)))
    assert c.run() == kara.KARA_E_INVAL


def test_stage_entry_points_validate():
    assert kara.lib.kara_topk(4, 0, 1, FAKE, FAKE, None) == kara.KARA_E_INVAL
    assert kara.lib.kara_topk(4, 10, 11, FAKE, FAKE, None) == kara.KARA_E_INVAL
    assert kara.lib.kara_topk(4, 3000, 1, FAKE, FAKE, None) == kara.KARA_E_INVAL
    assert kara.lib.kara_token2chunk(4, 10, 3, 11, FAKE, FAKE, FAKE, None) == kara.KARA_E_INVAL
    assert kara.lib.kara_token2chunk(-1, 10, 3, 5, FAKE, FAKE, FAKE, None) == kara.KARA_E_INVAL
    assert kara.lib.kara_topk(0, 10, 3, None, None, None) == kara.KARA_OK     # nothing to do


def test_schedule_worked_example():
    """Step 256 with period 128 and W=1024: seq 0 has 3000 fresh tokens (eligible), seq 1 only
    500 past its watermark, seq 2 is shorter than the window, seq 3 was not selected."""
    import torch
    lens = torch.tensor([3000, 5000, 900, 2048], dtype=torch.int32)
    wm = torch.tensor([0, 4500, 0, 0], dtype=torch.int32)
    sel = torch.tensor([1, 1, 1, 0], dtype=torch.uint8)
    assert kara.kara_schedule_step(256, 128, 1024, lens, wm, sel) == [0]
    assert kara.kara_schedule_step(200, 128, 1024, lens, wm, sel) == []     # not a period boundary
    assert kara.kara_schedule_step(0, 128, 1024, lens, wm, sel) == []


def test_schedule_matches_oracle():
    import numpy as np
    import torch

    from oracle import kara_oracle as ko
    rng = np.random.default_rng(3)
    for trial in range(50):
        n = int(rng.integers(0, 40))
        lens = rng.integers(1, 5000, size=n)
        wm = np.array([int(rng.integers(0, L + 1)) for L in lens], dtype=np.int64)
        sel = rng.random(n) < 0.5
        step = int(rng.integers(0, 1000))
        P = int(rng.integers(1, 200))
        W = int(rng.integers(1, 3000))
        want = ko.schedule_step(step, P, W, lens.tolist(), wm.tolist(), sel.tolist())
        got = kara.kara_schedule_step(step, P, W, torch.tensor(lens, dtype=torch.int32),
                                      torch.tensor(wm, dtype=torch.int32), torch.tensor(sel))
        assert got == want


def test_schedule_rejects():
    import torch
    lens = torch.tensor([100], dtype=torch.int32)
    with pytest.raises(kara.KaraError):
        kara.kara_schedule_step(128, 128, 10, lens, torch.tensor([101], dtype=torch.int32), torch.tensor([1]))
    with pytest.raises(kara.KaraError):
        kara.kara_schedule_step(128, 0, 10, lens, torch.tensor([0], dtype=torch.int32), torch.tensor([1]))


def test_compress_static_rejects_oversized_batch_before_side_effects():
    """The no-allocation entry point refuses a batch whose scratch need exceeds
    its static array, before reading any argument beyond shape and params."""
    sh, pr = shape(), params()
    assert kara.kara_static_scratch_bytes() == 256 << 20
    n = 1
    while kara.kara_workspace_bytes(sh, pr, n) <= kara.kara_static_scratch_bytes():
        n *= 2
    assert kara.kara_workspace_bytes(sh, pr, n) > kara.kara_static_scratch_bytes()
    pool = kara.Pool(20, list(range(20)))
    st = kara.lib.kara_compress_static(
        ctypes.byref(sh), ctypes.byref(pr), n, FAKE * 16, FAKE * 16, 20, FAKE, FAKE * 16, 5, FAKE, FAKE * 16,
        pool.handle, FAKE, FAKE * 16, FAKE, None, None, None, None, None)
    assert st == kara.KARA_E_WORKSPACE
    assert "static scratch" in kara.kara_last_error()
    assert pool.snapshot() == list(range(20))


def _ring(window, n_slots=2):
    return kara.kara_query_ring(FAKE * 16, n_slots, window, FAKE * 16, FAKE * 16)


def test_ring_window_must_match_the_call():
    """A query ring records the window it was built with; appending or
    compressing with another window is rejected before anything is touched
    (the ring's rows would otherwise be indexed past their end)."""
    sh = shape()
    ring = _ring(window=16)
    st = kara.lib.kara_append(ctypes.byref(sh), 8, 1, 0, FAKE * 16, FAKE * 16, FAKE * 16, FAKE * 16, 20,
                              FAKE * 16, 5, FAKE * 16, ctypes.byref(ring), None)
    assert st == kara.KARA_E_INVAL and "window" in kara.kara_last_error()
    c = Call()
    before = c.pool.snapshot()
    st = kara.lib.kara_compress_ring(
        ctypes.byref(c.shape), ctypes.byref(c.params), len(c.lens), ctypes.byref(_ring(window=c.params.window + 1)),
        FAKE * 16, c.n_blocks, c.table, FAKE * 16, c.max_blocks, _i32(c.lens), FAKE * 16, c.pool.handle,
        c.new_table, FAKE * 16, c.new_lens, 256 * 16, c.ws, None, None, None, None, None)
    assert st == kara.KARA_E_INVAL and "window" in kara.kara_last_error()
    assert c.pool.snapshot() == before
    assert list(c.new_lens) == [0, 0]


def test_plan_lengths_match_the_oracle_plan():
    """kara_plan_lengths (the library's own per-sequence plan) against the
    oracle's plan_compaction: new lengths and fresh blocks taken per sequence."""
    import numpy as np
    import torch

    from oracle import kara_oracle as ko
    rng = np.random.default_rng(11)
    for trial in range(30):
        bs = int(2 ** rng.integers(0, 7))
        W = int(rng.integers(1, 600))
        B = int(rng.integers(0, W))
        C = W - B
        R = int(rng.integers(1, C + 1))
        K = int(rng.integers(1, C + 1))
        lens = rng.integers(W, W + 3000, size=int(rng.integers(0, 12)))
        MB = int(max([-(-int(L) // bs) for L in lens] + [1])) + 8
        table = np.arange(len(lens) * MB).reshape(len(lens), MB)
        fifo = ko.FifoPool(range(10 ** 6, 10 ** 6 + 10 ** 5))
        want_table, want_lens = ko.plan_compaction(table, lens, W, B, R, bs, fifo)
        new_lens, fresh = kara.kara_plan_lengths(kara.kara_params(W, B, K, R), bs,
                                                  torch.tensor(lens, dtype=torch.int32))
        assert new_lens.tolist() == want_lens.tolist()
        taken = [int((row >= 10 ** 6).sum()) for row in want_table]
        assert fresh.tolist() == taken
    with pytest.raises(kara.KaraError):
        kara.kara_plan_lengths(kara.kara_params(8, 2, 2, 3), 3, torch.tensor([10], dtype=torch.int32))
    with pytest.raises(kara.KaraError):
        kara.kara_plan_lengths(kara.kara_params(8, 2, 2, 3), 4, torch.tensor([7], dtype=torch.int32))


def test_decode_attention_rejects_pools_beyond_32_bit_rows():
    """Decode attention numbers a layer's K rows in 32 bits: a pool with
    n_blocks * n_kv_heads * block_size >= 2^32 rows is refused before any
    pointer is read."""
    sh = shape(n_kv_heads=8, block_size=1024)
    lens = (ctypes.c_int32 * 1)(5)
    st = kara.lib.kara_decode_attention(ctypes.byref(sh), 1, 0, FAKE * 16, FAKE * 16, 1 << 19, FAKE * 16, 4,
                                        lens, FAKE * 16, FAKE * 16, FAKE * 16, 1 << 30, None)
    assert st == kara.KARA_E_UNSUPPORTED
    assert "2^32" in kara.kara_last_error()
