"""Pins of the oracle's Top-K and Token2Chunk: hand-worked examples, a
rank-count definition of Top-K, structural invariants of the chunk fill, and a
mutation test of the pins."""

import json
import os

import numpy as np
import pytest

from oracle import kara_oracle as ko

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _worked():
    with open(os.path.join(GOLD, "select_worked.json")) as f:
        return json.load(f)


def topk_by_rank(s, k):
    """Position j is a candidate iff fewer than k positions beat it (higher
    score, or equal score at a lower index)."""
    C = len(s)
    out = []
    for j in range(C):
        beaten_by = sum(1 for i in range(C) if s[i] > s[j] or (s[i] == s[j] and i < j))
        if beaten_by < k:
            out.append(j)
    return np.array(out)


def test_topk_worked():
    w = _worked()
    s = np.array(w["scores"], dtype=np.float64)
    for case in w["topk"]:
        assert ko.topk_candidates(s, case["k"]).tolist() == case["cand"], case["derivation"]


@pytest.mark.parametrize("dtype", [np.float32, np.float64])
@pytest.mark.parametrize("seed", range(6))
def test_topk_rank_definition(seed, dtype):
    rng = np.random.default_rng(seed)
    C = int(rng.integers(1, 60))
    k = int(rng.integers(1, C + 1))
    s = rng.integers(0, 5, size=C).astype(dtype) * dtype(0.25) if seed % 2 else rng.random(C).astype(dtype)
    assert ko.topk_candidates(s, k).tolist() == topk_by_rank(s, k).tolist()


def test_topk_flat_takes_lowest_indices():
    s = np.full(20, 3.0, dtype=np.float32)
    assert ko.topk_candidates(s, 5).tolist() == [0, 1, 2, 3, 4]


def test_topk_float32_decides_in_float32():
    # 1 + 2^-30 rounds to 1.0 in float32: the two entries tie, the lower index wins.
    s64 = np.array([1.0, 1.0 + 2.0 ** -30])
    assert ko.topk_candidates(s64, 1).tolist() == [1]
    assert ko.topk_candidates(s64.astype(np.float32), 1).tolist() == [0]


def test_t2c_worked():
    w = _worked()
    s = np.array(w["scores"], dtype=np.float64)
    for case in w["t2c"]:
        cand = ko.topk_candidates(s, case["k"])
        assert ko.token2chunk(s, cand, case["r"]).tolist() == case["retained"], case["derivation"]
        assert ko.token2chunk(s.astype(np.float32), cand, case["r"]).tolist() == case["retained"]


def check_t2c_invariants(s, k, r, t2c=ko.token2chunk, topk=ko.topk_candidates):
    """Structural facts the fill must satisfy, stated without its code."""
    C = len(s)
    cand = topk(s, k)
    kept, accepted = t2c(s, cand, r, return_spans=True)
    kept = np.asarray(kept)
    assert len(kept) == r
    assert np.all(np.diff(kept) > 0)
    assert kept.min() >= 0 and kept.max() < C
    if r < k:
        assert kept.tolist() == topk(s, r).tolist()
        return
    assert set(cand.tolist()) <= set(kept.tolist())
    # spans with a gap, ordered by (sigma desc, left endpoint asc)
    ft = np.asarray(s).dtype.type
    spans = []
    for a, b in zip(cand[:-1], cand[1:]):
        g = int(b - a - 1)
        if g:
            spans.append(((s[a] + s[b]) / ft(g + 2), int(a), int(b), g))
    spans.sort(key=lambda t: (-t[0], t[1]))
    prefix, expect = 0, []
    for sig, a, b, g in spans:
        if prefix + g > r - k:
            break
        prefix += g
        expect.append((a, b))
    assert [tuple(map(int, x)) for x in accepted] == expect
    keptset = set(kept.tolist())
    for a, b in accepted:
        assert set(range(a, b + 1)) <= keptset
    # the rest of the budget went to the best positions outside candidates and spans
    base = set(cand.tolist())
    for a, b in accepted:
        base |= set(range(a + 1, b))
    extra = sorted(keptset - base)
    outside = [j for j in range(C) if j not in base]
    best = sorted(outside, key=lambda j: (-s[j], j))[:len(extra)]
    assert sorted(best) == extra


@pytest.mark.parametrize("dtype", [np.float32, np.float64])
@pytest.mark.parametrize("seed", range(20))
def test_t2c_invariants_random(seed, dtype):
    rng = np.random.default_rng(100 + seed)
    C = int(rng.integers(4, 200))
    k = int(rng.integers(1, min(C, 40) + 1))
    r = int(rng.integers(1, C))
    kind = seed % 3
    if kind == 0:
        s = rng.random(C)
    elif kind == 1:
        s = rng.integers(0, 4, size=C) * 0.5
    else:
        s = np.where(rng.random(C) < 0.1, 5.0 + rng.random(C), rng.random(C) * 1e-3)
    check_t2c_invariants(s.astype(dtype), k, r)


def test_t2c_budget_equals_k_keeps_candidates():
    rng = np.random.default_rng(9)
    s = rng.random(50)
    cand = ko.topk_candidates(s, 10)
    assert ko.token2chunk(s, cand, 10).tolist() == cand.tolist()


def test_t2c_adjacent_candidates_make_no_span():
    s = np.array([5.0, 5.0, 0.1, 0.2, 0.3, 5.0])
    cand = ko.topk_candidates(s, 3)            # [0, 1, 5]
    kept, spans = ko.token2chunk(s, cand, 6, return_spans=True)
    assert spans == [(1, 5)] and kept.tolist() == [0, 1, 2, 3, 4, 5]


# ---------------------------------------------------------------------------
# Mutation test for the selection pins
# ---------------------------------------------------------------------------

def _t2c_mutant(kind):
    def f(scores, cand, budget, return_spans=False):
        s = np.asarray(scores)
        C = len(s)
        cand = [int(c) for c in cand]
        K = len(cand)
        if budget < K:
            out = ko.topk_candidates(s, budget)
            return (out, []) if return_spans else out
        ft = s.dtype.type
        spans = []
        for m in range(K - 1):
            a, b = cand[m], cand[m + 1]
            g = b - a - 1
            if g == 0:
                continue
            if kind == "sigma_mean_no_length":
                sig = (s[a] + s[b]) / ft(2)
            elif kind == "sigma_over_gap":
                sig = (s[a] + s[b]) / ft(g)
            else:
                sig = (s[a] + s[b]) / ft(g + 2)
            spans.append((sig, a, b, g))
        key = (lambda t: (t[0], t[1])) if kind == "ascending_sigma" else (lambda t: (-t[0], t[1]))
        spans.sort(key=key)
        room = budget - K
        kept = np.zeros(C, bool)
        kept[cand] = True
        used, acc = 0, []
        for sig, a, b, g in spans:
            if used + g > room:
                if kind == "skip_and_continue":
                    continue
                break
            used += g
            kept[a + 1:b] = True
            acc.append((a, b))
        need = budget - int(kept.sum())
        if kind == "no_topup":
            need = 0
        order = np.lexsort((np.arange(C), -s)) if kind != "topup_low_index" else np.arange(C)
        for j in order:
            if need == 0:
                break
            if not kept[j]:
                kept[j] = True
                need -= 1
        out = np.flatnonzero(kept)
        return (out, acc) if return_spans else out
    return f


def _t2c_pins(fn):
    w = _worked()
    s = np.array(w["scores"], dtype=np.float64)
    for case in w["t2c"]:
        cand = ko.topk_candidates(s, case["k"])
        assert fn(s, cand, case["r"]).tolist() == case["retained"]
    for seed in range(20):
        rng = np.random.default_rng(100 + seed)
        C = int(rng.integers(4, 200))
        k = int(rng.integers(1, min(C, 40) + 1))
        r = int(rng.integers(1, C))
        check_t2c_invariants(rng.random(C), k, r, t2c=fn)


def test_t2c_pins_accept_oracle():
    _t2c_pins(ko.token2chunk)


@pytest.mark.parametrize("kind", ["sigma_mean_no_length", "sigma_over_gap", "ascending_sigma",
                                  "skip_and_continue", "no_topup", "topup_low_index"])
def test_t2c_pins_reject_mutants(kind):
    with pytest.raises(AssertionError):
        _t2c_pins(_t2c_mutant(kind))
