"""GPU edge cases through the C ABI: an empty batch for every entry point, the
largest window and region the kernels support (W = 4096, C = 2048), and the
block-size extremes (1 and 1024 tokens per block), each end to end against
the oracle with the same bars as tests/test_gpu_parity.py."""

import pytest
import torch

from parity import oracle_scores

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from decode_kv_cache_kara_amd import kara, runner, synth
    from test_gpu_parity import check_e2e, run_e2e


def say(*a):
    print("[case]", *a, flush=True)


def test_empty_batch_does_nothing():
    say("empty batch")
    wl = synth.make_workload(0, device="cuda")
    shape = runner.shape_of(wl)
    params = runner.params_of(wl)
    pool = kara.Pool(wl.n_blocks, wl.free_ids)
    before = pool.snapshot()
    empty_i = torch.empty((0, wl.max_blocks), dtype=torch.int32)
    empty_l = torch.empty((0,), dtype=torch.int32)
    ws = torch.empty(256, dtype=torch.uint8, device="cuda")
    pool_bytes = wl.pool.clone()
    kara.kara_compress(shape, params, wl.q_window[:0], wl.pool, empty_i, empty_i.cuda(), empty_l, empty_l.cuda(),
                       pool, empty_i.clone(), empty_i.cuda(), empty_l.clone(), ws)
    kara.kara_decode_attention(shape, 0, wl.q_window[:0, 0, 0], wl.pool, empty_i.cuda(), empty_l, empty_l.cuda(),
                               torch.empty((0, wl.n_q_heads, wl.head_dim), device="cuda"), ws)
    ring = kara.QueryRing(torch.zeros((1, wl.n_layers, wl.window, wl.n_q_heads, wl.head_dim), dtype=wl.dtype,
                                      device="cuda"), empty_l.cuda(), empty_l.cuda())
    kara.kara_append(shape, wl.window, -1, wl.q_window[:0, :, 0], wl.pool[0, 0, :0, :, 0], wl.pool[0, 0, :0, :, 0],
                     wl.pool, empty_i.cuda(), empty_l.cuda(), ring)
    torch.cuda.synchronize()
    assert pool.snapshot() == before
    assert torch.equal(wl.pool, pool_bytes)


EDGE_CASES = {
    # the largest window and region: 4096 window tokens, 2048 compressible,
    # 32 row chunks per unit, 64 key tiles per pass
    "max-window-4096-region-2048": dict(n_seqs=2, n_layers=1, n_q_heads=4, n_kv_heads=1, head_dim=128,
                                        block_size=16, window=4096, protect=2048, top_k=256, budget=700,
                                        lens=[4096, 5003], dtype=torch.bfloat16, qk_std=0.3),
    # one token per block: every window row in its own block
    "block-size-1": dict(n_seqs=2, n_layers=2, n_q_heads=4, n_kv_heads=2, head_dim=128, block_size=1,
                         window=96, protect=16, top_k=10, budget=30, lens=[96, 211], dtype=torch.bfloat16,
                         qk_std=0.5),
    # 1024 tokens per block: the window spans at most two blocks
    "block-size-1024": dict(n_seqs=3, n_layers=1, n_q_heads=8, n_kv_heads=2, head_dim=64, block_size=1024,
                            window=700, protect=60, top_k=20, budget=100, lens=[700, 1500, 3000],
                            dtype=torch.bfloat16, qk_std=0.5),
}


@pytest.mark.parametrize("name", list(EDGE_CASES))
def test_edge_end_to_end(name):
    say("edge end to end", name)
    wl = synth.make_workload(None, device="cuda", **EDGE_CASES[name])
    orc = oracle_scores(wl)
    ses, pool, before = run_e2e(wl)
    verdicts = check_e2e(wl, ses, pool, before, orc, case=f"edge {name}")
    say(name, verdicts)


@pytest.fixture(autouse=True)
def _release_memory():
    yield
    import gc
    gc.collect()
    if torch.cuda.is_available():
        torch.cuda.empty_cache()
