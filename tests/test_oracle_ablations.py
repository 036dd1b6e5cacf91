"""Pins of the oracle's two ablations (Technical Summary: Kara, Experimental
Results, Ablation Studies): unidirectional window scoring, where query i only
sees keys j <= i, and Token2Chunk off, where the kept set is the top-R set.

Unidirectional scores are pinned by closed forms (two-token windows, identical
keys giving harmonic sums), a pure-Python brute force, a library attention
routine (torch's causal scaled-dot-product attention applied to an identity
value matrix returns the attention matrix itself), the mass invariant and the
causality invariant (queries before key j do not change its score).  A mutation
test checks that these pins catch the plausible mistakes: the mask transposed,
the diagonal excluded, the mask applied after normalisation."""

import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import kara_oracle as ko

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def logistic(x):
    return 1.0 / (1.0 + math.exp(-x))


def harmonic(n):
    return sum(1.0 / m for m in range(1, n + 1))


# ---------------------------------------------------------------------------
# Unidirectional scoring
# ---------------------------------------------------------------------------

def uni(q, k, protect):
    return ko.window_scores(q, k, protect, unidirectional=True)


def two_token_case(fn):
    """W = 2, one head, D = 1: row 0 sees key 0 only (weight 1); row 1 weighs
    key 0 by logistic(q1 (k0 - k1))."""
    q = np.array([[[1.0]], [[2.0]]])
    k = np.array([[[1.0]], [[0.0]]])
    s = fn(q, k, 0)
    want = np.array([[1.0 + logistic(2.0), 1.0 - logistic(2.0)]])
    np.testing.assert_allclose(s, want, rtol=1e-14, atol=0)
    # D = 4 with the 1/sqrt(D) scale: logit difference q1 . (k0 - k1) / 2
    rng = np.random.default_rng(11)
    q = rng.normal(size=(2, 1, 4))
    k = rng.normal(size=(2, 1, 4))
    d = float(q[1, 0] @ (k[0, 0] - k[1, 0])) / 2.0
    np.testing.assert_allclose(fn(q, k, 1), np.array([[1.0 + logistic(d)]]), rtol=1e-14, atol=0)


def harmonic_case(fn):
    """Identical keys (or zero queries): row i is uniform over its i + 1 keys,
    so s_j = G * (H_W - H_j)."""
    rng = np.random.default_rng(12)
    W, Hq, Hkv, D, B = 8, 6, 2, 4, 3
    want = np.array([[3.0 * (harmonic(W) - harmonic(j)) for j in range(W - B)]] * Hkv)
    k = np.broadcast_to(rng.normal(size=(1, Hkv, D)), (W, Hkv, D))
    np.testing.assert_allclose(fn(rng.normal(size=(W, Hq, D)), k, B), want, rtol=1e-13)
    np.testing.assert_allclose(fn(np.zeros((W, Hq, D)), rng.normal(size=(W, Hkv, D)), B), want,
                               rtol=1e-13)


def brute_force_uni(q, k, protect):
    """Pure-Python loops with math.exp; row i runs over keys 0..i only."""
    W, Hq, D = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    C = W - protect
    out = [[0.0] * C for _ in range(Hkv)]
    for qh in range(Hq):
        h = qh // G
        for i in range(W):
            logits = []
            for j in range(i + 1):
                dot = 0.0
                for d in range(D):
                    dot += float(q[i, qh, d]) * float(k[j, h, d])
                logits.append(dot / math.sqrt(D))
            m = max(logits)
            ex = [math.exp(x - m) for x in logits]
            tot = sum(ex)
            for j in range(min(i + 1, C)):
                out[h][j] += ex[j] / tot
    return np.array(out)


def library_uni(q, k, protect):
    """torch's causal attention with V = identity returns the attention rows."""
    W, Hq, D = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    qt = torch.tensor(q).permute(1, 0, 2)                          # [Hq, W, D]
    kt = torch.tensor(k).permute(1, 0, 2).repeat_interleave(G, 0)  # [Hq, W, D]
    v = torch.eye(W, dtype=torch.float64).expand(Hq, W, W)
    p = torch.nn.functional.scaled_dot_product_attention(qt, kt, v, is_causal=True)  # [Hq, W, W]
    return p.sum(dim=1).reshape(Hkv, G, W).sum(dim=1)[:, :W - protect].numpy()


def test_uni_closed_forms():
    two_token_case(uni)
    harmonic_case(uni)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_uni_brute_force(seed):
    rng = np.random.default_rng(seed)
    W, Hq, Hkv, D, B = 7, 6, 2, 5, 2
    q = rng.normal(size=(W, Hq, D))
    k = rng.normal(size=(W, Hkv, D))
    np.testing.assert_allclose(uni(q, k, B), brute_force_uni(q, k, B), rtol=1e-12, atol=0)


def test_uni_library_attention():
    rng = np.random.default_rng(5)
    W, Hq, Hkv, D, B = 33, 8, 2, 16, 5
    q = rng.normal(size=(W, Hq, D))
    k = rng.normal(size=(W, Hkv, D))
    np.testing.assert_allclose(uni(q, k, B), library_uni(q, k, B), rtol=1e-12, atol=1e-15)


def causality_and_mass(fn):
    rng = np.random.default_rng(8)
    W, Hq, Hkv, D = 13, 4, 2, 6
    q = rng.normal(size=(W, Hq, D)) * 2
    k = rng.normal(size=(W, Hkv, D)) * 2
    s = fn(q, k, 0)
    np.testing.assert_allclose(s.sum(axis=1), np.full(Hkv, 2.0 * W), rtol=1e-12)
    j = 6
    q2 = q.copy()
    q2[:j] = rng.normal(size=(j, Hq, D)) * 2        # queries before key j change
    np.testing.assert_allclose(fn(q2, k, 0)[:, j:], s[:, j:], rtol=1e-12)


def test_uni_invariants():
    causality_and_mass(uni)


def test_uni_differs_from_bidirectional():
    rng = np.random.default_rng(9)
    q = rng.normal(size=(9, 4, 8))
    k = rng.normal(size=(9, 2, 8))
    assert not np.allclose(uni(q, k, 2), ko.window_scores(q, k, 2), rtol=1e-3)


def _uni_mutant(kind):
    def f(q_win, k_win, protect):
        q = np.asarray(q_win, dtype=np.float64)
        k = np.asarray(k_win, dtype=np.float64)
        W, Hq, D = q.shape
        Hkv = k.shape[1]
        G = Hq // Hkv
        s = np.zeros((Hkv, W - protect))
        mask = {"transposed_mask": np.triu(np.ones((W, W), bool)),
                "strict": np.tril(np.ones((W, W), bool), -1)}.get(kind, np.tril(np.ones((W, W), bool)))
        with np.errstate(invalid="ignore"):
            for qh in range(Hq):
                x = (q[:, qh] @ k[:, qh // G].T) / np.sqrt(D)
                if kind == "mask_after_softmax":
                    e = np.exp(x - x.max(axis=1, keepdims=True))
                    p = np.where(mask, e / e.sum(axis=1, keepdims=True), 0.0)
                else:
                    x = np.where(mask, x, -np.inf)
                    e = np.exp(x - x.max(axis=1, keepdims=True))
                    p = e / e.sum(axis=1, keepdims=True)
                s[qh // G] += p[:, :W - protect].sum(axis=0)
        return s
    return f


def _all_uni_pins(fn):
    two_token_case(fn)
    harmonic_case(fn)
    rng = np.random.default_rng(1)
    q = rng.normal(size=(7, 6, 5))
    k = rng.normal(size=(7, 2, 5))
    np.testing.assert_allclose(fn(q, k, 2), brute_force_uni(q, k, 2), rtol=1e-12)
    causality_and_mass(fn)


def test_uni_pins_accept_the_oracle():
    _all_uni_pins(uni)


@pytest.mark.parametrize("kind", ["transposed_mask", "strict", "mask_after_softmax"])
def test_uni_pins_reject_mutants(kind):
    with pytest.raises(AssertionError):
        _all_uni_pins(_uni_mutant(kind))


# ---------------------------------------------------------------------------
# Token2Chunk off
# ---------------------------------------------------------------------------

def test_no_chunks_worked_examples():
    with open(os.path.join(GOLD, "select_worked.json")) as f:
        g = json.load(f)
    s = np.array(g["scores"], dtype=np.float32)
    for case in g["no_chunks"]:
        for k in (1, 4, 5):
            got = ko.select_retained(s, min(k, case["r"]), case["r"], chunks=False)
            assert got.tolist() == case["retained"], (case, k)


@pytest.mark.parametrize("seed", [0, 1, 2, 3])
def test_no_chunks_is_top_r_by_sorting(seed):
    """Against a plain Python sort of (-score, position) pairs."""
    rng = np.random.default_rng(seed)
    C = 40
    s = rng.integers(0, 6, size=C).astype(np.float32)   # many ties
    for R in (1, 7, 20, 40):
        want = sorted(j for _, j in sorted((-float(s[j]), j) for j in range(C))[:R])
        assert ko.select_retained(s, 5, R, chunks=False).tolist() == want


def test_compress_flags_reach_every_stage():
    """End to end on a tiny paged workload: the ablation flags change scores
    and kept sets exactly as the stage functions say."""
    rng = np.random.default_rng(3)
    S, Lyr, W, Hq, Hkv, D, bs, B, K, R = 2, 2, 16, 4, 2, 8, 4, 4, 3, 6
    lens = np.array([20, 23])
    nb = 24
    pool = rng.normal(size=(Lyr, 2, nb, Hkv, bs, D))
    perm = rng.permutation(nb)
    table = np.full((S, 8), -1, dtype=np.int64)
    table[0, :5] = perm[:5]
    table[1, :6] = perm[5:11]
    free = [int(x) for x in perm[11:]]
    q = rng.normal(size=(S, Lyr, W, Hq, D))
    for uni_flag in (False, True):
        for chunks in (True, False):
            out = ko.compress(q, pool, table, lens, W, B, K, R, bs, free,
                              unidirectional=uni_flag, chunks=chunks)
            for b in range(S):
                for l in range(Lyr):
                    kw = ko.window_keys(pool, table[b], int(lens[b]), W, l, Hkv, bs)
                    s = ko.window_scores(q[b, l], kw, B, unidirectional=uni_flag)
                    np.testing.assert_array_equal(out["scores"][b, l], s)
                    for h in range(Hkv):
                        want = ko.select_retained(s[h], K, R, chunks=chunks)
                        assert out["retained"][b, l, h].tolist() == want.tolist()
