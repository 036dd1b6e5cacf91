"""Plain CPU definition of the serving-policy simulation: periodic window
compression against threshold-triggered whole-cache compression, under a KV
memory cap and a concurrency limit.

TEST INFRASTRUCTURE ONLY: imported by tests; never by the product path.

Sources: "Technical Summary: Kara", Problem Statement 1 (threshold
triggering lowers throughput as concurrency grows) and Methodology 3 (the
periodic policy); paper, Fig. 1 caption (compression frees memory so more
sequences decode at once).  The pages give no simulation; the step rules
below are this library's reading, written out one rule at a time:

  1. admission: waiting requests enter in order while fewer than max_batch
     run and the free pool holds the prompt's blocks plus one spare block;
  2. decode: each running sequence in admission order appends one token,
     taking a new block when its length is a multiple of the block size; with
     no free block it stalls for the step; if every running sequence stalled,
     the most recently admitted one is preempted: its blocks are freed and it
     goes back to the front of the queue, to restart from its prompt;
  3. sequences that generated all their tokens leave and free their blocks;
  4. compression (none for the uncompressed baseline): periodic - at multiples of the period, running sequences
     with length - watermark >= W go from L to L - (W - B) + R tokens, their
     tail from block (L - W) // bs on held in ceil(((L - W) % bs + R + B) / bs)
     blocks, watermark = new length - B; threshold - running sequences with
     length >= threshold keep `keep` tokens (ceil(keep / bs) blocks);
  5. step time = fixed + per_token * (cached tokens of the sequences running
     when the step's decode starts) + compression cost (periodic: a constant
     per sequence; threshold: a constant per cached key scored).

Request i generates gen_min + splitmix64(seed + i) % (gen_max - gen_min + 1)
tokens, with SplitMix64 as published by Steele, Lea and Flood (2014).
"""

from math import ceil

MASK = (1 << 64) - 1


def splitmix64(x):
    """One SplitMix64 output for state x (the state is advanced by the golden
    gamma 0x9e3779b97f4a7c15 first, then mixed)."""
    z = (x + 0x9E3779B97F4A7C15) & MASK
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & MASK
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & MASK
    return z ^ (z >> 31)


def gen_length(cfg, i):
    return cfg["gen_min"] + splitmix64((cfg["seed"] + i) & MASK) % (cfg["gen_max"] - cfg["gen_min"] + 1)


def simulate(cfg):
    """Returns (summary dict, per-step list of (running after the step,
    compressions in the step, step time)).  The summary's `admissions` lists
    request ids in admission order, re-admissions after a preemption
    included."""
    bs = cfg["block_size"]
    free = cfg["cap_blocks"]
    running = []           # dicts: req, len, left, gen, wm, blocks
    waiting = list(range(cfg["n_requests"]))
    steps = []
    admissions = []
    tokens = stalls = compressions = peak = preemptions = wasted = 0
    total_ms = compress_ms = 0.0
    step = 0
    while step < cfg["max_steps"] and (waiting or running):
        step += 1
        while waiting and len(running) < cfg["max_batch"]:
            need = ceil(cfg["prompt_len"] / bs)
            if free < need + 1:
                break
            free -= need
            req = waiting.pop(0)
            admissions.append(req)
            running.append(dict(req=req, len=cfg["prompt_len"], left=gen_length(cfg, req), gen=0, wm=0,
                                blocks=need))
        ms = cfg["decode_ms_fixed"] + cfg["decode_ms_per_token"] * sum(s["len"] for s in running)
        advanced = 0
        for s in running:
            if s["len"] % bs == 0:
                if free < 1:
                    stalls += 1
                    continue
                free -= 1
                s["blocks"] += 1
            s["len"] += 1
            s["left"] -= 1
            s["gen"] += 1
            tokens += 1
            advanced += 1
        if running and advanced == 0:
            victim = running.pop()
            free += victim["blocks"]
            wasted += victim["gen"]
            preemptions += 1
            waiting.insert(0, victim["req"])
        for s in [s for s in running if s["left"] <= 0]:
            free += s["blocks"]
        running = [s for s in running if s["left"] > 0]
        n_comp = 0
        c_ms = 0.0
        if cfg["policy"] == "periodic":
            W, B, R = cfg["window"], cfg["protect"], cfg["budget"]
            if step % cfg["period"] == 0:
                for s in running:
                    if s["len"] - s["wm"] < W:
                        continue
                    after = (s["len"] - W) // bs + ceil(((s["len"] - W) % bs + R + B) / bs)
                    free += s["blocks"] - after
                    s["blocks"] = after
                    s["len"] = s["len"] - (W - B) + R
                    s["wm"] = s["len"] - B
                    c_ms += cfg["compress_ms_per_seq"]
                    n_comp += 1
        elif cfg["policy"] == "threshold":
            for s in running:
                if s["len"] < cfg["threshold"]:
                    continue
                c_ms += cfg["compress_ms_per_key"] * s["len"]
                after = ceil(cfg["keep"] / bs)
                free += s["blocks"] - after
                s["blocks"] = after
                s["len"] = cfg["keep"]
                n_comp += 1
        ms += c_ms
        compressions += n_comp
        compress_ms += c_ms
        peak = max(peak, cfg["cap_blocks"] - free)
        total_ms += ms
        steps.append((len(running), n_comp, ms))
    summary = dict(steps=step, tokens=tokens, compressions=compressions, stalls=stalls, peak_blocks=peak,
                   preemptions=preemptions, wasted=wasted,
                   finished=cfg["n_requests"] - len(running) - len(waiting), total_ms=total_ms,
                   compress_ms=compress_ms,
                   mean_active=(sum(a for a, _, _ in steps) / step) if step else 0.0, admissions=admissions)
    return summary, steps
