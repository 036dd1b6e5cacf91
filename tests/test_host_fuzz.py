"""Property test of the C ABI's front end (no GPU): for random kara_compress
(and kara_paged_compact) arguments, valid or not, a non-OK status leaves the block pool unchanged, and
every status but KARA_E_HIP also leaves the host outputs untouched, with a
message from kara_last_error().  On a machine without a GPU every call ends
non-OK (an argument error, or KARA_E_HIP at the first device call), so the
whole contract is exercised.  The device pointers are placeholders that are
never dereferenced without a device; the test does not run where a GPU is
visible."""

import ctypes

import pytest
import torch
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

from decode_kv_cache_kara_amd import kara

FAKE = 0x100                    # 16- and 256-byte aligned, never dereferenced
SENTINEL = -7

pytestmark = pytest.mark.skipif(torch.cuda.device_count() > 0,
                                reason="placeholder device pointers: only where no GPU is visible")


MUTATIONS = ["short-sequence", "duplicate-block", "block-out-of-range", "hole-in-table", "few-free-blocks",
             "free-block-in-table", "short-workspace", "no-workspace", "max-blocks-too-small", "top-k-above-region",
             "budget-zero", "unknown-flag", "bad-heads", "bad-block-size", "bad-head-dim", "protect-equals-window"]


@st.composite
def calls(draw):
    """A valid call, then up to two mutations that each break one rule."""
    Lyr = draw(st.integers(1, 2))
    Hkv = draw(st.integers(1, 2))
    G = draw(st.integers(1, 3))
    D = draw(st.sampled_from([64, 128]))
    bs = draw(st.sampled_from([1, 2, 4, 16]))
    dtype = draw(st.sampled_from([kara.KARA_F32, kara.KARA_BF16]))
    W = draw(st.integers(4, 24))
    B = draw(st.integers(0, W - 1))
    C = W - B
    K = draw(st.integers(1, C))
    R = draw(st.integers(1, C))
    n = draw(st.integers(1, 3))
    lens = [draw(st.integers(W, W + 40)) for _ in range(n)]
    nblk = [-(-L // bs) for L in lens]
    max_blocks = max(nblk) + draw(st.integers(0, 2))
    fresh = sum(-(-((L - W) % bs + R + B) // bs) for L in lens)
    n_blocks = sum(nblk) + fresh + draw(st.integers(0, 6))
    perm = draw(st.permutations(list(range(n_blocks))))
    table, cur = [], 0
    for L, k in zip(lens, nblk):
        table += perm[cur:cur + k] + [-1] * (max_blocks - k)
        cur += k
    free = perm[cur:]
    shape = [Lyr, G * Hkv, Hkv, D, bs, dtype]
    params = [W, B, K, R, 0]
    ws_kind = "exact"
    n_mut = draw(st.sampled_from([1, 2, 1, 0, 1]))
    for m in draw(st.lists(st.sampled_from(MUTATIONS), min_size=n_mut, max_size=n_mut)):
        if m == "short-sequence":
            lens[0] = W - 1
        elif m == "duplicate-block" and nblk[0] >= 1 and n > 1:
            table[max_blocks] = table[0]
        elif m == "block-out-of-range":
            table[0] = n_blocks + 3
        elif m == "hole-in-table" and nblk[0] >= 2:
            table[1] = -1
        elif m == "few-free-blocks":
            free = free[:max(fresh - 1, 0)]
        elif m == "free-block-in-table" and free:
            table[0] = free[0]
        elif m == "short-workspace":
            ws_kind = "short"
        elif m == "no-workspace":
            ws_kind = "none"
        elif m == "max-blocks-too-small" and max(nblk) > 1:
            max_blocks_new = max(nblk) - 1
            table = [x for b in range(n) for x in table[b * max_blocks:b * max_blocks + max_blocks_new]]
            max_blocks = max_blocks_new
        elif m == "top-k-above-region":
            params[2] = C + 1
        elif m == "budget-zero":
            params[3] = 0
        elif m == "unknown-flag":
            params[4] = 4
        elif m == "bad-heads":
            shape[1] = G * Hkv + 1
        elif m == "bad-block-size":
            shape[4] = 3
        elif m == "bad-head-dim":
            shape[3] = 96
        elif m == "protect-equals-window":
            params[1] = W
    return dict(shape=tuple(shape), params=tuple(params), lens=lens, max_blocks=max_blocks, n_blocks=n_blocks,
                table=table, free=free, ws_kind=ws_kind)


def _i32(vals):
    return (ctypes.c_int32 * max(len(vals), 1))(*vals)


@settings(max_examples=400, deadline=None, suppress_health_check=[HealthCheck.too_slow])
@given(calls())
def test_failed_calls_change_nothing(c):
    shape = kara.kara_shape(*c["shape"])
    params = kara.kara_params(*c["params"])
    n = len(c["lens"])
    try:
        pool = kara.Pool(c["n_blocks"], c["free"])
    except kara.KaraError:
        return                                   # the pool itself is invalid; nothing to call
    before = pool.snapshot()
    ws_need = kara.kara_workspace_bytes(shape, params, n)
    ws = {"exact": ws_need, "short": max(ws_need - 256, 0), "none": 0}[c["ws_kind"]]
    new_table = _i32([SENTINEL] * (n * c["max_blocks"]))
    new_lens = _i32([SENTINEL] * n)
    st_ = kara.lib.kara_compress(
        ctypes.byref(shape), ctypes.byref(params), n, FAKE, FAKE, c["n_blocks"], _i32(c["table"]), FAKE,
        c["max_blocks"], _i32(c["lens"]), FAKE, pool.handle, new_table, FAKE, new_lens,
        FAKE if ws else None, ws, None, None, None, None, None)
    if st_ == kara.KARA_OK:
        assert n == 0                            # only an empty batch succeeds without a device
        return
    assert kara.kara_last_error()
    assert pool.snapshot() == before
    if st_ != kara.KARA_E_HIP:
        assert list(new_lens)[:n] == [SENTINEL] * n
        assert list(new_table)[:n * c["max_blocks"]] == [SENTINEL] * (n * c["max_blocks"])


@settings(max_examples=300, deadline=None, suppress_health_check=[HealthCheck.too_slow])
@given(calls())
def test_failed_compaction_calls_change_nothing(c):
    """The same contract for the compaction stage's own entry point."""
    shape = kara.kara_shape(*c["shape"])
    params = kara.kara_params(*c["params"])
    n = len(c["lens"])
    try:
        pool = kara.Pool(c["n_blocks"], c["free"])
    except kara.KaraError:
        return
    before = pool.snapshot()
    new_table = _i32([SENTINEL] * (n * c["max_blocks"]))
    new_lens = _i32([SENTINEL] * n)
    st_ = kara.lib.kara_paged_compact(
        ctypes.byref(shape), ctypes.byref(params), n, FAKE, c["n_blocks"], _i32(c["table"]), FAKE,
        c["max_blocks"], _i32(c["lens"]), FAKE, FAKE, pool.handle, new_table, FAKE, new_lens, None)
    if st_ == kara.KARA_OK:
        assert n == 0
        return
    assert kara.kara_last_error()
    assert pool.snapshot() == before
    if st_ != kara.KARA_E_HIP:
        assert list(new_lens)[:n] == [SENTINEL] * n
        assert list(new_table)[:n * c["max_blocks"]] == [SENTINEL] * (n * c["max_blocks"])
