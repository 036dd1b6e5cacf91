"""Serving-policy comparison on the native simulator (kara_policy_sim):
periodic window compression, threshold-triggered whole-cache compression and
no compression, over a seeded reasoning-trace workload with Distill-Llama-8B
cache geometry, under a KV memory cap, for several concurrency limits.

The per-step costs are measured on the GPU by the caller (bench.py):
  decode_ms_per_token   decode attention per cached token and layer, times
                        the layers (the model's weight reads are the fixed
                        per-step part, an input);
  compress_ms_per_seq   one kara_compress of one sequence (all layers);
  compress_ms_per_key   a whole-cache scoring pass per cached key, taken as
                        the window step's cost per window key (the scoring
                        kernel's cost grows with the keys it scores).
"""

from __future__ import annotations

from . import kara

# Workload: 512 requests, prompts of 512 tokens, reasoning traces of 4k-16k
# generated tokens, 16-token blocks, a KV budget of 400k tokens (about 52 GB
# of Distill-Llama-8B cache).
WORKLOAD = dict(n_requests=512, block_size=16, prompt_len=512, gen_min=4096, gen_max=16384, seed=2024,
                cap_blocks=25_000, max_steps=2_000_000)
PERIODIC = dict(policy="periodic", window=1024, protect=128, budget=179, period=128, threshold=0, keep=0)
# threshold policy: a sequence's whole cache is compressed to 2048 tokens when
# it reaches 4096 (a footprint close to the periodic policy's at these lengths)
THRESHOLD = dict(policy="threshold", window=0, protect=0, budget=0, period=1, threshold=4096, keep=2048)
NONE = dict(policy="none", window=0, protect=0, budget=0, period=1, threshold=0, keep=0)


def compare(costs, batches=(32, 64, 128, 256, 512)):
    """Rows of (policy, max_batch, summary) for each concurrency limit."""
    rows = []
    for mb in batches:
        for pol in (PERIODIC, THRESHOLD, NONE):
            cfg = dict(WORKLOAD, **pol, **costs, max_batch=mb)
            summary, _ = kara.kara_policy_sim(cfg)
            useful = summary["tokens"] - summary["wasted"]
            summary["tokens_per_s"] = useful / (summary["total_ms"] / 1e3) if summary["total_ms"] else 0.0
            summary["compress_share"] = summary["compress_ms"] / summary["total_ms"] if summary["total_ms"] else 0.0
            rows.append((pol["policy"], mb, summary))
    return rows
