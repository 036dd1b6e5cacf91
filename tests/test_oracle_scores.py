"""Pins of the oracle's window scoring against things other than itself:
closed forms, exact special cases, an invariant, an independent pure-Python
brute force and a library softmax.  A mutation test checks that the pins catch
the plausible mistakes (wrong scale, transposed operand, causal mask, softmax
over the region only, protected queries dropped, interleaved GQA mapping)."""

import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import kara_oracle as ko

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _golden_cases():
    with open(os.path.join(GOLD, "scores_closed_form.json")) as f:
        return json.load(f)["cases"]


def check_golden(fn):
    for c in _golden_cases():
        s = fn(np.array(c["q"]), np.array(c["k"]), c["protect"])
        np.testing.assert_allclose(s, np.array(c["scores"]), rtol=0, atol=1e-14, err_msg=c["name"])


def brute_force(q, k, protect):
    """Pure-Python loops with math.exp: row softmax over all W keys, column sums."""
    W, Hq, D = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    C = W - protect
    out = [[0.0] * C for _ in range(Hkv)]
    for qh in range(Hq):
        h = qh // G
        for i in range(W):
            logits = []
            for j in range(W):
                dot = 0.0
                for d in range(D):
                    dot += float(q[i, qh, d]) * float(k[j, h, d])
                logits.append(dot / math.sqrt(D))
            m = max(logits)
            ex = [math.exp(x - m) for x in logits]
            tot = sum(ex)
            for j in range(C):
                out[h][j] += ex[j] / tot
    return np.array(out)


def test_closed_forms():
    check_golden(ko.window_scores)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_brute_force_tiny(seed):
    rng = np.random.default_rng(seed)
    W, Hq, Hkv, D, B = 7, 6, 2, 5, 2
    q = rng.normal(size=(W, Hq, D))
    k = rng.normal(size=(W, Hkv, D))
    np.testing.assert_allclose(ko.window_scores(q, k, B), brute_force(q, k, B), rtol=1e-12, atol=0)


def test_library_softmax():
    """Against torch's CPU softmax in float64 (a different library routine)."""
    rng = np.random.default_rng(5)
    W, Hq, Hkv, D, B = 33, 8, 2, 16, 5
    q = rng.normal(size=(W, Hq, D))
    k = rng.normal(size=(W, Hkv, D))
    G = Hq // Hkv
    qt = torch.tensor(q).permute(1, 0, 2)                    # [Hq, W, D]
    kt = torch.tensor(k).permute(1, 0, 2).repeat_interleave(G, 0)
    p = torch.softmax(torch.matmul(qt, kt.transpose(1, 2)) / math.sqrt(D), dim=-1)   # [Hq, W, W]
    ref = p.sum(dim=1).reshape(Hkv, G, W).sum(dim=1)[:, :W - B].numpy()
    np.testing.assert_allclose(ko.window_scores(q, k, B), ref, rtol=1e-12, atol=0)


def test_uniform_special_cases():
    """Zero queries or identical keys make every row uniform: s_j = G exactly."""
    rng = np.random.default_rng(3)
    W, Hq, Hkv, D, B = 8, 6, 2, 4, 3
    q = np.zeros((W, Hq, D))
    k = rng.normal(size=(W, Hkv, D))
    np.testing.assert_allclose(ko.window_scores(q, k, B), np.full((Hkv, W - B), 3.0), rtol=1e-15)
    q = rng.normal(size=(W, Hq, D))
    k = np.broadcast_to(rng.normal(size=(1, Hkv, D)), (W, Hkv, D))
    np.testing.assert_allclose(ko.window_scores(q, k, B), np.full((Hkv, W - B), 3.0), rtol=1e-14)


def test_mass_invariant():
    """With no protected buffer, the scores of a head sum to G * W (each row sums to 1)."""
    rng = np.random.default_rng(4)
    W, Hq, Hkv, D = 19, 12, 4, 8
    q = rng.normal(size=(W, Hq, D)) * 2
    k = rng.normal(size=(W, Hkv, D)) * 2
    s = ko.window_scores(q, k, 0)
    np.testing.assert_allclose(s.sum(axis=1), np.full(Hkv, 3 * W), rtol=1e-13)


def test_permutation_equivariance():
    """Bidirectional scoring has no position bias: permuting the window permutes the scores."""
    rng = np.random.default_rng(6)
    W, Hq, Hkv, D = 11, 4, 2, 6
    q = rng.normal(size=(W, Hq, D))
    k = rng.normal(size=(W, Hkv, D))
    perm = rng.permutation(W)
    s = ko.window_scores(q, k, 0)
    sp = ko.window_scores(q[perm], k[perm], 0)
    np.testing.assert_allclose(sp, s[:, perm], rtol=1e-13)


def test_protected_buffer_is_a_prefix_cut():
    """Scores of the region do not depend on B beyond truncation."""
    rng = np.random.default_rng(7)
    W, Hq, Hkv, D = 12, 4, 4, 3
    q = rng.normal(size=(W, Hq, D))
    k = rng.normal(size=(W, Hkv, D))
    full = ko.window_scores(q, k, 0)
    np.testing.assert_allclose(ko.window_scores(q, k, 5), full[:, :7], rtol=1e-15)


# ---------------------------------------------------------------------------
# Mutation test: each planted mistake must fail at least one pin.
# ---------------------------------------------------------------------------

def _mutant(kind):
    def f(q_win, k_win, protect):
        q = np.asarray(q_win, dtype=np.float64)
        k = np.asarray(k_win, dtype=np.float64)
        W, Hq, D = q.shape
        Hkv = k.shape[1]
        G = Hq // Hkv
        C = W - protect
        s = np.zeros((Hkv, C))
        scale = {"no_scale": 1.0, "scale_1_over_D": 1.0 / D}.get(kind, 1.0 / np.sqrt(D))
        for qh in range(Hq):
            h = (qh % Hkv) if kind == "interleaved_gqa" else qh // G
            x = (q[:, qh] @ k[:, h].T) * scale
            if kind == "transposed":
                x = x.T
            if kind == "causal":
                x = np.where(np.tril(np.ones((W, W), bool)), x, -np.inf)
            if kind == "region_softmax":
                x = x[:, :C]
            e = np.exp(x - x.max(axis=1, keepdims=True))
            p = e / e.sum(axis=1, keepdims=True)
            rows = slice(0, C) if kind == "drop_protected_queries" else slice(0, W)
            if kind == "sign":
                p = np.exp(-(x - x.max(axis=1, keepdims=True)))
                p = p / p.sum(axis=1, keepdims=True)
            s[h] += p[rows, :C].sum(axis=0)
        return s
    return f


def _all_pins(fn):
    check_golden(fn)
    rng = np.random.default_rng(1)
    W, Hq, Hkv, D, B = 7, 6, 2, 5, 2
    q = rng.normal(size=(W, Hq, D))
    k = rng.normal(size=(W, Hkv, D))
    np.testing.assert_allclose(fn(q, k, B), brute_force(q, k, B), rtol=1e-12)
    perm = rng.permutation(W)
    np.testing.assert_allclose(fn(q[perm], k[perm], 0), fn(q, k, 0)[:, perm], rtol=1e-12)
    np.testing.assert_allclose(fn(q, k, 0).sum(axis=1), np.full(Hkv, 3 * W), rtol=1e-12)


def test_pins_accept_the_oracle():
    _all_pins(ko.window_scores)


@pytest.mark.parametrize("kind", ["no_scale", "scale_1_over_D", "interleaved_gqa", "transposed",
                                  "causal", "region_softmax", "drop_protected_queries", "sign"])
def test_pins_reject_mutants(kind):
    with pytest.raises(AssertionError):
        _all_pins(_mutant(kind))
