"""The serving-policy simulator: the oracle pinned by closed forms and by
SplitMix64's published outputs, and the native simulator (kara_policy_sim)
equal to the oracle, step by step, on seeded random settings.  Host code
only; runs without a GPU."""

import numpy as np
import pytest

from decode_kv_cache_kara_amd import kara
from oracle import policy_oracle as po


def base(**kw):
    cfg = dict(policy="periodic", n_requests=1, max_batch=4, cap_blocks=10_000, block_size=16, prompt_len=100,
               gen_min=50, gen_max=50, seed=0, window=128, protect=16, budget=24, period=1, threshold=0, keep=0,
               decode_ms_fixed=2.0, decode_ms_per_token=1e-3, compress_ms_per_seq=0.5, compress_ms_per_key=1e-3,
               max_steps=100_000)
    cfg.update(kw)
    return cfg


def test_splitmix64_published_outputs():
    # the first two outputs of the generator started from state 0
    assert po.splitmix64(0) == 0xE220A8397B1DCDAF
    assert po.splitmix64(0x9E3779B97F4A7C15) == 0x6E789E6AA1B965F4


def test_one_request_without_compression():
    """Five tokens, nothing to compress: steps = 5 and the decode cost is
    a sum over lengths prompt .. prompt + 4."""
    cfg = base(gen_min=5, gen_max=5, window=1000, budget=24)
    s, steps = po.simulate(cfg)
    assert (s["steps"], s["tokens"], s["compressions"], s["finished"]) == (5, 5, 0, 1)
    want = 5 * 2.0 + 1e-3 * sum(100 + t for t in range(5))
    assert abs(s["total_ms"] - want) < 1e-12
    assert [a for a, _, _ in steps] == [1, 1, 1, 1, 0]


@pytest.mark.parametrize("gen", [28, 29, 113, 114, 500])
def test_periodic_one_sequence_closed_form(gen):
    """Prompt of exactly W tokens, period 1: the first token makes the window
    eligible; afterwards the window refills every W - B tokens.  A sequence
    that finishes on a step leaves before compression, so the compressions
    fall on steps 1 + k (W - B) < gen."""
    W, B, R = 128, 16, 24
    cfg = base(prompt_len=W, gen_min=gen, gen_max=gen, window=W, protect=B, budget=R)
    s, steps = po.simulate(cfg)
    want = [1 + k * (W - B) for k in range(gen) if 1 + k * (W - B) < gen]
    assert [i + 1 for i, (_, c, _) in enumerate(steps) if c] == want
    assert s["compressions"] == len(want) and s["compress_ms"] == pytest.approx(0.5 * len(want))


@pytest.mark.parametrize("gen", [30, 31, 90, 200])
def test_threshold_one_sequence_closed_form(gen):
    """Prompt P < T: first compression after T - P tokens, then every T - keep."""
    P, T, keep = 100, 130, 64
    cfg = base(policy="threshold", prompt_len=P, gen_min=gen, gen_max=gen, threshold=T, keep=keep)
    s, steps = po.simulate(cfg)
    n = 0 if gen <= T - P else 1 + (gen - 1 - (T - P)) // (T - keep)
    assert s["compressions"] == n
    # each compression scores T keys
    assert abs(s["compress_ms"] - n * T * 1e-3) < 1e-12


def test_sequential_service_with_one_slot():
    cfg = base(n_requests=6, max_batch=1, gen_min=10, gen_max=40, seed=3, window=10_000)
    s, steps = po.simulate(cfg)
    total = sum(po.gen_length(cfg, i) for i in range(6))
    assert s["steps"] == total and s["tokens"] == total and s["finished"] == 6
    assert max(a for a, _, _ in steps) == 1


def test_memory_cap_stalls_and_preemption():
    """Twelve long requests in 40 blocks: without compression the running
    sequences exhaust the pool, stall, and the newest is preempted until the
    rest can finish; every request still finishes and the cap holds."""
    cfg = base(n_requests=12, max_batch=12, cap_blocks=40, gen_min=200, gen_max=300, seed=5, window=10_000)
    s, _ = po.simulate(cfg)
    assert s["peak_blocks"] <= 40
    assert s["stalls"] > 0 and s["preemptions"] > 0
    assert s["finished"] == 12
    assert s["tokens"] == sum(po.gen_length(cfg, i) for i in range(12)) + s["wasted"]
    # periodic compression frees blocks: fewer preemptions, less waste
    s2, _ = po.simulate(dict(cfg, window=64, protect=8, budget=12, period=8))
    assert s2["finished"] == 12 and s2["wasted"] < s["wasted"]


def test_rule_request_lengths_cover_the_range():
    """gen_min + x % (gen_max - gen_min + 1): over 200 requests every length
    from gen_min to gen_max occurs, and none outside."""
    cfg = base(gen_min=7, gen_max=10, seed=123)
    assert {po.gen_length(cfg, i) for i in range(200)} == {7, 8, 9, 10}


def test_rule_blocks_follow_the_length():
    """One request, no compression: a block is taken whenever a token is
    appended at a length that is a multiple of the block size, so after a step
    the sequence holds ceil(length / bs) blocks.  The peak is read at the end
    of a step, after finished sequences left, so it is the count at the end of
    the second-to-last step, length prompt + gen - 1 (none for gen = 1).
    Lengths on both sides of block boundaries."""
    for prompt, gen in [(16, 2), (16, 17), (16, 18), (17, 16), (17, 17), (5, 12), (5, 13), (16, 1)]:
        cfg = base(prompt_len=prompt, gen_min=gen, gen_max=gen, window=10_000)
        s, _ = po.simulate(cfg)
        want = -(-(prompt + gen - 1) // 16) if gen > 1 else 0
        assert s["peak_blocks"] == want, (prompt, gen)


def test_rule_periodic_new_length():
    """Prompt of W tokens, period 1, gen 50 < W - B: one compression, at step
    1, from W + 1 tokens to (W + 1) - (W - B) + R; step k >= 2 then starts
    with B + R + k - 1 tokens.  The total time is the sum of the step costs."""
    W, B, R, g = 128, 16, 24, 50
    cfg = base(prompt_len=W, gen_min=g, gen_max=g, window=W, protect=B, budget=R)
    s, _ = po.simulate(cfg)
    cached = W + sum(B + R + k - 1 for k in range(2, g + 1))
    assert s["compressions"] == 1
    assert abs(s["total_ms"] - (g * 2.0 + 1e-3 * cached + 0.5)) < 1e-9


def test_rule_preempted_request_returns_to_the_front():
    """Block size 1, prompt 1, 4 blocks, 2 slots, 3 requests of 3 tokens
    (traced by hand from the rules): step 1 admits 0 and 1 (2 blocks left,
    both append); step 2 both stall, 1 (the newest) is preempted and goes back
    to the front; step 3 re-admits 1, only 0 appends; step 4 both stall and 1
    is preempted again; step 5 admits nobody (one free block, one spare
    needed), 0 finishes; step 6 admits 1, then 2."""
    cfg = base(policy="none", n_requests=3, max_batch=2, cap_blocks=4, block_size=1, prompt_len=1,
               gen_min=3, gen_max=3, window=10_000)
    s, steps = po.simulate(cfg)
    assert s["admissions"][:5] == [0, 1, 1, 1, 2]
    assert s["preemptions"] >= 2 and s["finished"] == 3
    assert [a for a, _, _ in steps[:5]] == [2, 1, 2, 1, 0]


@pytest.mark.parametrize("seed", range(8))
@pytest.mark.parametrize("policy", ["periodic", "threshold", "none"])
def test_native_simulator_equals_oracle(policy, seed):
    rng = np.random.default_rng(seed)
    bs = int(rng.choice([4, 16]))
    W = int(rng.integers(32, 160))
    B = int(rng.integers(0, W // 4))
    cfg = base(policy=policy, n_requests=int(rng.integers(1, 40)), max_batch=int(rng.integers(1, 16)),
               cap_blocks=int(rng.integers(60, 400)), block_size=bs, prompt_len=int(rng.integers(20, 200)),
               gen_min=int(rng.integers(20, 100)), gen_max=int(rng.integers(100, 600)), seed=int(rng.integers(1 << 40)),
               window=W, protect=B, budget=int(rng.integers(1, W - B + 1)), period=int(rng.integers(1, 64)),
               threshold=int(rng.integers(250, 400)), keep=int(rng.integers(40, 200)),
               decode_ms_fixed=float(rng.random()), decode_ms_per_token=float(rng.random() * 1e-3),
               compress_ms_per_seq=float(rng.random()), compress_ms_per_key=float(rng.random() * 1e-3),
               max_steps=20_000)
    a, sa = kara.kara_policy_sim(cfg)
    b, sb = po.simulate(cfg)
    for k in ("steps", "tokens", "compressions", "stalls", "peak_blocks", "preemptions", "wasted", "finished"):
        assert a[k] == b[k], k
    assert [x[:2] for x in sa] == [x[:2] for x in sb]
    np.testing.assert_allclose([x[2] for x in sa], [x[2] for x in sb], rtol=1e-12)
    for k in ("total_ms", "compress_ms", "mean_active"):
        assert abs(a[k] - b[k]) <= 1e-9 * max(1.0, abs(b[k])), k
    assert [kara.kara_sim_gen_length(cfg, i) for i in range(5)] == [po.gen_length(cfg, i) for i in range(5)]


@pytest.mark.parametrize("policy", ["periodic", "threshold", "none"])
def test_native_simulator_equals_oracle_under_memory_pressure(policy):
    cfg = base(policy=policy, n_requests=30, max_batch=20, cap_blocks=90, block_size=16, prompt_len=60,
               gen_min=100, gen_max=500, seed=11, window=96, protect=8, budget=16, period=16, threshold=300,
               keep=100, max_steps=50_000)
    a, sa = kara.kara_policy_sim(cfg)
    b, sb = po.simulate(cfg)
    assert b["preemptions"] > 0 and b["stalls"] > 0
    for k in ("steps", "tokens", "compressions", "stalls", "peak_blocks", "preemptions", "wasted", "finished"):
        assert a[k] == b[k], k
    assert [x[:2] for x in sa] == [x[:2] for x in sb]


def test_native_simulator_rejects():
    with pytest.raises(kara.KaraError):
        kara.kara_policy_sim(base(max_batch=0))
    with pytest.raises(kara.KaraError):
        kara.kara_policy_sim(base(policy="threshold", threshold=50, keep=60))
    with pytest.raises(kara.KaraError):
        kara.kara_policy_sim(base(cap_blocks=3))          # the prompt alone needs 7 + 1 blocks
