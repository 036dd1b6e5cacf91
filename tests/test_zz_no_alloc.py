"""kara_compress_static, the entry point for callers that cannot allocate
device memory, against kara_compress with a caller workspace: both run the
same kernels on the same inputs, so scores, candidates, kept sets, the
compacted cache, tables, lengths and the free list must agree bit for bit.
Two calls in a row share the library's static scratch, the second on a
smaller batch."""

import numpy as np
import pytest
import torch

from parity import bits

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from decode_kv_cache_kara_amd import kara, runner, synth


def _static_call(wl, ses, outputs):
    pool = ses.new_pool()
    nt_h = torch.empty_like(ses.table_h)
    nt_d = torch.empty_like(ses.table_d)
    nl_h = torch.empty_like(ses.lens_h)
    U, C = wl.n_units, wl.region
    outs = dict(scores=None, cand=None, retained=None)
    if outputs:
        outs = dict(scores=torch.full((U, C), float("nan"), device="cuda"),
                    cand=torch.full((U, wl.top_k), -7, dtype=torch.int32, device="cuda"),
                    retained=torch.full((U, wl.budget), -7, dtype=torch.int32, device="cuda"))
    kara.kara_compress_static(ses.shape, ses.params, wl.q_window, wl.pool, ses.table_h, ses.table_d, ses.lens_h,
                              ses.lens_d, pool, nt_h, nt_d, nl_h, scores_out=outs["scores"],
                              cand_out=outs["cand"], retained_out=outs["retained"])
    torch.cuda.synchronize()
    return pool, nt_h, nt_d, nl_h, outs


def _check_against_workspace_call(wl, outputs):
    ses = runner.Session(wl)
    assert kara.kara_workspace_bytes(ses.shape, ses.params, wl.n_seqs) <= kara.kara_static_scratch_bytes()
    before = wl.pool.clone()
    ref_pool = ses.compress()
    torch.cuda.synchronize()
    ref_cache = wl.pool.clone()
    wl.pool.copy_(before)
    torch.cuda.synchronize()
    pool, nt_h, nt_d, nl_h, outs = _static_call(wl, ses, outputs)
    assert torch.equal(bits(wl.pool), bits(ref_cache))
    assert nt_h.tolist() == ses.new_table_h.tolist()
    assert nt_d.cpu().tolist() == ses.new_table_d.cpu().tolist()
    assert nl_h.tolist() == ses.new_lens_h.tolist()
    assert pool.snapshot() == ref_pool.snapshot()
    if outputs:
        assert torch.equal(bits(outs["scores"]), bits(ses.scores))
        assert torch.equal(outs["cand"], ses.cand)
        assert torch.equal(outs["retained"], ses.retained)
    # the compaction really moved rows (the test is not vacuous)
    assert not torch.equal(bits(wl.pool), bits(before))


def test_static_scratch_matches_workspace_call_twice():
    print("[case] static scratch: Qwen3-4B-shaped 4 seqs x 4 layers, then 2 seqs x 1 layer", flush=True)
    big = synth.make_workload(2, device="cuda", n_seqs=4, n_layers=4)
    _check_against_workspace_call(big, outputs=True)
    del big
    print("[case] static scratch: second, smaller call", flush=True)
    small = synth.make_workload(None, device="cuda", n_seqs=2, n_layers=1, n_q_heads=8, n_kv_heads=2,
                                head_dim=128, block_size=16, window=200, protect=13, top_k=12, budget=40,
                                lens=(200, 700), dtype=torch.bfloat16, qk_std=0.25)
    _check_against_workspace_call(small, outputs=False)


def test_static_scratch_two_key_block_windows():
    """A 2048-key window (the scorer's three launches keep per-row normaliser
    inputs and per-unit flags in the scratch too), after the one-block calls
    above have left other contents in it."""
    print("[case] static scratch: Qwen3-14B-shaped 2 seqs x 2 layers, W=2048", flush=True)
    wl = synth.make_workload(3, device="cuda", n_seqs=2, n_layers=2)
    _check_against_workspace_call(wl, outputs=True)


def test_static_scratch_rejects_oversized_calls():
    print("[case] static scratch: oversized call rejected", flush=True)
    wl = synth.make_workload(2, device="cuda", n_seqs=2, n_layers=1)
    ses = runner.Session(wl)
    # a batch whose scratch need exceeds the array (the lengths tensor sets
    # n_seqs; the workspace's segments are padded, so the need is not linear in n)
    n = 1
    while kara.kara_workspace_bytes(ses.shape, ses.params, n) <= kara.kara_static_scratch_bytes():
        n *= 2
    lens_h = torch.full((n,), int(ses.lens_h[0]), dtype=torch.int32)
    table_h = ses.table_h[:1].repeat(n, 1).contiguous()
    pool = ses.new_pool()
    before = wl.pool.clone()
    with pytest.raises(kara.KaraError) as e:
        kara.kara_compress_static(ses.shape, ses.params, wl.q_window, wl.pool, table_h, ses.table_d, lens_h,
                                  ses.lens_d, pool, torch.empty_like(table_h), ses.new_table_d,
                                  torch.empty_like(lens_h))
    assert e.value.status == kara.KARA_E_WORKSPACE
    assert "static scratch" in str(e.value)
    torch.cuda.synchronize()
    assert torch.equal(bits(wl.pool), bits(before))
    assert pool.snapshot() == ses.new_pool().snapshot()
