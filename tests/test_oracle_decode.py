"""Pins of the oracle's decode-side functions: the window's query states
(the last W produced, in order) and decode attention over a paged cache,
against torch's scaled-dot-product attention (a library routine), closed
forms (one cached token gives its V row; identical keys give the mean of V)
and the paged gather (a shuffled block table gives the same result as a
contiguous one)."""

import math

import numpy as np
import pytest
import torch

from oracle import kara_oracle as ko


def paged(rng, Lyr, Hkv, D, L, bs, extra=5):
    """A pool holding one sequence of L tokens in shuffled blocks, plus the
    contiguous K/V it holds, [Lyr, 2, L, Hkv, D]."""
    nb = -(-L // bs) + extra
    pool = rng.normal(size=(Lyr, 2, nb, Hkv, bs, D))
    table = rng.permutation(nb)[: -(-L // bs)]
    kv = np.stack([np.stack([np.stack([pool[l, c, table[t // bs], :, t % bs] for t in range(L)])
                             for c in range(2)]) for l in range(Lyr)])
    return pool, table, kv


def test_window_queries_are_the_last_w_in_order():
    hist = [np.full((2, 3, 4), float(n)) for n in range(10)]
    w = ko.window_queries(hist, 4)
    assert w.shape == (2, 4, 3, 4)
    assert [float(w[0, i, 0, 0]) for i in range(4)] == [6.0, 7.0, 8.0, 9.0]
    with pytest.raises(ValueError):
        ko.window_queries(hist[:3], 4)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_decode_attention_matches_library(seed):
    rng = np.random.default_rng(seed)
    Lyr, Hq, Hkv, D, L, bs = 2, 8, 2, 16, 37, 4
    pool, table, kv = paged(rng, Lyr, Hkv, D, L, bs)
    q = rng.normal(size=(Hq, D)) * 1.5
    for l in range(Lyr):
        got = ko.decode_attention(q, pool, table, L, l, bs)
        G = Hq // Hkv
        qt = torch.tensor(q).reshape(Hq, 1, D)
        kt = torch.tensor(kv[l, 0]).permute(1, 0, 2).repeat_interleave(G, 0)   # [Hq, L, D]
        vt = torch.tensor(kv[l, 1]).permute(1, 0, 2).repeat_interleave(G, 0)
        want = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt).reshape(Hq, D).numpy()
        np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-13)


def test_decode_attention_closed_forms():
    rng = np.random.default_rng(4)
    Lyr, Hq, Hkv, D, bs = 1, 4, 2, 8, 4
    pool, table, kv = paged(rng, Lyr, Hkv, D, 1, bs)
    q = rng.normal(size=(Hq, D))
    out = ko.decode_attention(q, pool, table, 1, 0, bs)
    for g in range(Hq):                          # one token: its V row
        np.testing.assert_allclose(out[g], kv[0, 1, 0, g // 2], rtol=1e-15)
    pool, table, kv = paged(rng, Lyr, Hkv, D, 11, bs)
    for t in range(11):                          # identical keys: the mean of V
        pool[0, 0, table[t // bs], :, t % bs] = pool[0, 0, table[0], :, 0]
    out = ko.decode_attention(q, pool, table, 11, 0, bs)
    for g in range(Hq):
        np.testing.assert_allclose(out[g], kv[0, 1, :, g // 2].mean(axis=0), rtol=1e-13)


def test_decode_attention_ignores_block_placement():
    rng = np.random.default_rng(5)
    Lyr, Hq, Hkv, D, L, bs = 1, 6, 3, 8, 21, 4
    pool, table, kv = paged(rng, Lyr, Hkv, D, L, bs)
    q = rng.normal(size=(Hq, D))
    nb = -(-L // bs)
    flat = np.zeros((Lyr, 2, nb, Hkv, bs, D))
    for t in range(L):
        flat[:, :, t // bs, :, t % bs] = kv[:, :, t]
    np.testing.assert_allclose(ko.decode_attention(q, pool, table, L, 0, bs),
                               ko.decode_attention(q, flat, np.arange(nb), L, 0, bs), rtol=1e-14)
