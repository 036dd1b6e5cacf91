"""The adjudicator accepts the oracle's own results and rejects clear errors."""

import numpy as np
import pytest

from oracle import kara_oracle as ko
from parity import adjudicate


@pytest.mark.parametrize("seed", range(10))
def test_adjudicator_accepts_oracle(seed):
    rng = np.random.default_rng(seed)
    C = int(rng.integers(10, 300))
    K = int(rng.integers(1, min(C, 40)))
    R = int(rng.integers(1, C))
    s = rng.random(C)
    cand = ko.topk_candidates(s, K)
    X = ko.token2chunk(s, cand, R)
    assert adjudicate(s, K, R, X, cand) == "exact"


@pytest.mark.parametrize("seed", range(10))
def test_adjudicator_rejects_swaps(seed):
    rng = np.random.default_rng(50 + seed)
    C, K, R = 120, 8, 30
    s = rng.random(C) + 0.5
    cand = ko.topk_candidates(s, K)
    X = ko.token2chunk(s, cand, R).tolist()
    # swap the worst kept non-candidate for the best dropped position
    kept_nc = [j for j in X if j not in set(cand.tolist())]
    out = [j for j in range(C) if j not in set(X)]
    a = min(kept_nc, key=lambda j: s[j])
    b = max(out, key=lambda j: s[j])
    s2 = s.copy()
    s2[b] = s[a] * 0.5   # make the dropped one clearly worse in the judged scores ...
    s2[a] = 3.0          # ... and the kept one clearly the best: X now drops a top position
    assert adjudicate(s2, K, R, X, cand).startswith("fail")


def test_adjudicator_accepts_near_tie():
    s = np.array([1.0, 5.0, 2.0, 2.0, 7.0, 1.0, 0.5, 6.0, 3.0, 3.0, 0.25, 0.25, 4.0, 8.0, 1.5, 5.0])
    # K=4: positions 1 and 15 tie at 5.0; taking 15 instead of 1 is a near-tie
    cand = [4, 7, 13, 15]
    X = ko.token2chunk(s, np.array(cand), 4)
    assert adjudicate(s, 4, 4, X, cand) == "near_tie"


def test_adjudicator_no_chunks():
    """Token2Chunk-off ablation: the kept set must be a top-R set."""
    s = np.array([1.0, 5.0, 2.0, 2.0, 7.0, 1.0, 0.5, 6.0, 3.0, 3.0, 0.25, 0.25, 4.0, 8.0, 1.5, 5.0])
    cand = [1, 4, 7, 13]
    top9 = [1, 2, 4, 7, 8, 9, 12, 13, 15]
    assert adjudicate(s, 4, 9, top9, cand, chunks=False) == "exact"
    # positions 2 and 3 tie at 2.0: the other one is a near-tie
    assert adjudicate(s, 4, 9, [1, 3, 4, 7, 8, 9, 12, 13, 15], cand, chunks=False) == "near_tie"
    # dropping 12 (4.0) for 14 (1.5) is not a top-R set
    assert adjudicate(s, 4, 9, [1, 2, 4, 7, 8, 9, 13, 14, 15], cand, chunks=False).startswith("fail")
    # the Token2Chunk result is not what the ablation keeps
    t2c = ko.token2chunk(s, np.array(cand), 9)
    assert adjudicate(s, 4, 9, t2c, cand, chunks=False).startswith("fail")
