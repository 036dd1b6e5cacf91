"""Mutation tests of the oracle's remaining pins: a plausible mistake planted
in Top-K, the compaction plan, the compaction copy, the window gather, decode
attention or the periodic schedule must make at least one of that function's
pins (test_oracle_select, test_oracle_compact, test_oracle_decode) fail.  The
mutants are patched into the oracle module, so pins that reach the function
through compress() see them too."""

from math import ceil

import numpy as np
import pytest

import test_oracle_compact as tc
import test_oracle_decode as tdec
import test_oracle_select as tsel
from oracle import kara_oracle as ko

# ---------------------------------------------------------------- pins per function


def _topk_pins():
    tsel.test_topk_worked()
    for seed in range(6):
        for dtype in (np.float32, np.float64):
            tsel.test_topk_rank_definition(seed, dtype)
    tsel.test_topk_flat_takes_lowest_indices()
    tsel.test_topk_float32_decides_in_float32()


def _compaction_pins():
    tc.test_worked_block_example()
    for seed in range(8):
        tc.test_tag_gather(seed)
        tc.test_pool_conservation_and_untouched_blocks(seed)
    tc.test_fifo_order()
    tc.test_pool_exhaustion_changes_nothing()
    tc.test_kv_bytes_of_the_pages()
    tc.test_end_to_end_tiny_consistent()
    for seed in range(4):
        tc.test_window_keys_tags(seed)


def _decode_pins():
    for seed in range(3):
        tdec.test_decode_attention_matches_library(seed)
    tdec.test_decode_attention_closed_forms()
    tdec.test_decode_attention_ignores_block_placement()


def _schedule_pins():
    tc.test_schedule_worked_example_oracle()


# ---------------------------------------------------------------- mutants


def _topk(kind):
    def f(scores, k):
        s = np.asarray(scores)
        idx = np.arange(s.shape[0])
        if kind == "ties-to-higher-index":
            order = np.lexsort((-idx, -s))
        elif kind == "lowest-scores":
            order = np.lexsort((idx, s))
        else:
            order = np.lexsort((idx, -s))
        if kind == "one-short":
            return np.sort(order[:k - 1])
        if kind == "unsorted":
            return order[:k]
        return np.sort(order[:k])
    return f


def _plan(kind):
    def f(table, lens, window, protect, budget, block_size, pool):
        table = np.asarray(table)
        S, MB = table.shape
        bs = block_size
        C = window - protect
        plans = []
        for b in range(S):
            L = int(lens[b])
            start = L - window
            f0 = start // bs
            p = start - f0 * bs
            if kind == "fresh-count-ignores-offset":
                n_new = ceil((budget + protect) / bs)
            else:
                n_new = ceil((p + budget + protect) / bs)
            if kind == "keeps-boundary-block":
                f0 += 1
            plans.append((L, f0, n_new))
        if sum(n for _, _, n in plans) > len(pool):
            raise ko.PoolExhausted("not enough free blocks")
        new_table = np.full((S, MB), -1, dtype=np.int64)
        new_lens = np.zeros(S, dtype=np.int64)
        for b, (L, f0, n_new) in enumerate(plans):
            new_table[b, :f0] = table[b, :f0]
            new_table[b, f0:f0 + n_new] = pool.pop(n_new)
            new_lens[b] = L - window + budget if kind == "length-drops-protected" else L - C + budget
        for b, (L, f0, n_new) in enumerate(plans):
            pool.push(table[b, f0 + (1 if kind == "leaks-boundary-block" else 0):ceil(L / bs)])
        return new_table, new_lens
    return f


def _apply(kind):
    def f(pool_arr, table, lens, new_table, window, protect, budget, block_size, retained):
        out = pool_arr.copy()
        Lyr, _, _, Hkv, bs, _ = pool_arr.shape
        for b in range(len(lens)):
            L = int(lens[b])
            start = L - window
            f0 = start // bs
            lead = [] if kind == "drops-boundary-prefix" else list(range(f0 * bs, start))
            for l in range(Lyr):
                for h in range(Hkv):
                    off = 0 if kind == "kept-not-offset" else start
                    kept = [off + int(j) for j in retained[b, l, h]]
                    tail = list(range(L - protect - 1, L - 1)) if kind == "protected-shifted" else \
                        list(range(L - protect, L))
                    order = lead + kept + tail
                    for kv in range(2):
                        src_kv = 0 if kind == "v-from-k" else kv
                        for n, t in enumerate(order):
                            dst = new_table[b, f0 + n // bs]
                            out[l, kv, dst, h, n % bs] = pool_arr[l, src_kv, table[b][t // bs], h, t % bs]
        return out
    return f


def _window_keys(kind):
    def f(pool_arr, table_row, length, window, layer, n_kv_heads, block_size):
        start = length - window + (1 if kind == "start-off-by-one" else 0)
        kv = 1 if kind == "reads-values" else 0
        rows = []
        for i in range(window):
            t = min(start + i, length - 1)
            rows.append(np.stack([pool_arr[layer, kv, table_row[t // block_size], h, t % block_size]
                                  for h in range(n_kv_heads)]))
        return np.stack(rows)
    return f


def _decode(kind):
    def f(q, pool_arr, table_row, length, layer, block_size):
        q = np.asarray(q, dtype=np.float64)
        Hq, D = q.shape
        Hkv = pool_arr.shape[3]
        G = Hq // Hkv
        out = np.zeros((Hq, D))
        for g in range(Hq):
            h = g % Hkv if kind == "interleaved-groups" else g // G
            k = ko.logical_tokens(pool_arr, table_row, length, layer, 0, h, block_size).astype(np.float64)
            v = ko.logical_tokens(pool_arr, table_row, length, 0 if kind == "values-of-layer-0" else layer,
                                  1, h, block_size).astype(np.float64)
            x = k @ q[g] if kind == "no-scale" else (k @ q[g]) / np.sqrt(D)
            e = np.exp(x - x.max())
            out[g] = (e / e.sum()) @ v
        return out
    return f


def _schedule(kind):
    def f(step, period, window, lens, watermarks, selected):
        if (step <= 0 and kind != "fires-at-step-0") or step % period:
            return []
        out = []
        for b in range(len(lens)):
            room = lens[b] - watermarks[b]
            eligible = room > window if kind == "strict-window" else room >= window
            if eligible and (selected[b] or kind == "ignores-selection"):
                out.append(b)
        return out
    return f


MUTANTS = {
    "topk_candidates": (_topk, _topk_pins, ["ties-to-higher-index", "lowest-scores", "one-short", "unsorted"]),
    "plan_compaction": (_plan, _compaction_pins, ["fresh-count-ignores-offset", "keeps-boundary-block",
                                                 "leaks-boundary-block", "length-drops-protected"]),
    "apply_compaction": (_apply, _compaction_pins, ["drops-boundary-prefix", "kept-not-offset",
                                                   "protected-shifted", "v-from-k"]),
    "window_keys": (_window_keys, _compaction_pins, ["start-off-by-one", "reads-values"]),
    "decode_attention": (_decode, _decode_pins, ["interleaved-groups", "values-of-layer-0", "no-scale"]),
    "schedule_step": (_schedule, _schedule_pins, ["fires-at-step-0", "strict-window", "ignores-selection"]),
}

CASES = [(fn, kind) for fn, (_, _, kinds) in MUTANTS.items() for kind in kinds]


@pytest.mark.parametrize("fn", list(MUTANTS))
def test_pins_pass_on_the_oracle(fn):
    MUTANTS[fn][1]()


@pytest.mark.parametrize("fn,kind", CASES)
def test_pins_reject_mutant(fn, kind, monkeypatch):
    make, pins, _ = MUTANTS[fn]
    monkeypatch.setattr(ko, fn, make(kind))
    with pytest.raises(AssertionError):
        pins()
