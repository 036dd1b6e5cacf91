"""Plain CPU definition of Kara's decode-time compression step.

TEST INFRASTRUCTURE ONLY: imported by tests, the smoke check and the CPU
baseline of the benchmark; never by the product path (see package header).

What is computed, per sequence b, layer l and KV head h (a "unit"):

  window     the trailing W tokens of the sequence, local index i = 0..W-1
             [Summary, Methodology 1, opening sentence and Mechanism];
  region     the compressible region is local keys j < C = W - B; the last B
             tokens form the protected buffer [Summary, Methodology 1,
             Mechanism];
  scores     s[j] = sum over the G query heads of KV head h and over all W
             window queries of softmax_j'(q . k_j' / sqrt(D))[j], the softmax
             running over all W window keys with no causal mask
             [Summary, Methodology 1, Mechanism and Rationale; Paper, Abstract];
  top-K      the K largest s, ties to the lower index, ascending
             [Summary, Methodology 1, Selection];
  chunks     consecutive candidates bound spans, each span scored from its
             length and its endpoint scores, spans accepted greedily into the
             budget [Summary, Methodology 2, Process and Outcome];
  compact    the kept rows are written into fresh blocks of the paged cache and
             the old trailing blocks are returned to the free pool
             [Summary, Methodology 3, Periodic Compression Policy].

Readings fixed here where the pages are silent (each one is also stated in the
repository's design notes):

  * softmax scale 1/sqrt(D); query head q belongs to KV head q // G;
  * chunk score sigma = (s[a] + s[b]) / (g + 2) for endpoints a < b with
    g = b - a - 1 interior tokens; spans ordered by sigma descending, ties to
    the lower left endpoint; the longest prefix of that order whose interior
    lengths fit in R - K is accepted (prefix greedy);
  * the budget R counts kept tokens of the compressible region, candidates
    included; after the chunks, the highest-scored remaining tokens top the
    set up to exactly R (ties to the lower index); if R < K the result is the
    top-R set;
  * compaction keeps the boundary block's leading tokens that precede the
    window, then the R kept tokens, then the B protected tokens, in order, in
    fresh blocks popped from a FIFO free list (sequences in call order); the
    old blocks from the boundary block to the old end are pushed to the back
    of the list after all fresh blocks are taken.

The chunk-score formula is this library's own reading (the pages leave it open), so the
Token2Chunk result is pinned against that stated formula only; parity with
the paper's unpublished formula is unpinned.

Ablations [Summary, Experimental Results, Ablation Studies: removing the
bidirectional scoring or the Token2Chunk module each costs accuracy]:

  * unidirectional scoring: window query i takes its softmax over window keys
    j <= i only (the causal attention the model itself computes), so key j
    is scored by the queries at and after it; everything else is unchanged;
  * Token2Chunk off: the kept set is the top-R set of the region (isolated
    pairs, ties to the lower index), i.e. the candidates are never expanded.
"""

from __future__ import annotations

from collections import deque
from math import ceil

import numpy as np


# ----------------------------------------------------------------------------
# Scoring  [Summary, Methodology 1, Mechanism / Rationale]
# ----------------------------------------------------------------------------

def window_scores(q_win, k_win, protect, unidirectional=False):
    """Bidirectional window attention scores of the compressible region.

    q_win: [W, Hq, D] window query states (any float dtype; upcast to float64).
    k_win: [W, Hkv, D] window key states.
    protect: B, the length of the protected buffer at the end of the window.
    unidirectional: the ablation; row i's softmax runs over keys j <= i only.
    Returns s: float64 [Hkv, C] with C = W - B.

    For every KV head h and every query head q of its group (q // G == h), every
    window query row i takes a softmax over ALL W window keys (no causal mask:
    queries also attend to later tokens), and the probabilities that land on
    keys j < C are added into s[h, j].
    """
    q = np.asarray(q_win, dtype=np.float64)
    k = np.asarray(k_win, dtype=np.float64)
    W, Hq, D = q.shape
    Wk, Hkv, Dk = k.shape
    if Wk != W or Dk != D or Hq % Hkv != 0:
        raise ValueError("shape mismatch between window queries and keys")
    C = W - protect
    if not 0 < C <= W:
        raise ValueError("protected buffer must leave a non-empty region")
    if not (np.all(np.isfinite(q)) and np.all(np.isfinite(k))):
        raise ValueError("non-finite window states")
    G = Hq // Hkv
    scale = 1.0 / np.sqrt(D)
    s = np.zeros((Hkv, C), dtype=np.float64)
    for h in range(Hkv):
        keys = k[:, h, :]                          # [W, D]
        for g in range(G):
            queries = q[:, h * G + g, :]           # [W, D]
            logits = (queries @ keys.T) * scale    # row i: query i, column j: key j
            if unidirectional:                     # keys after the query are not seen
                logits = np.where(np.tril(np.ones((W, W), dtype=bool)), logits, -np.inf)
            logits = logits - logits.max(axis=1, keepdims=True)
            e = np.exp(logits)
            p = e / e.sum(axis=1, keepdims=True)   # row softmax over the keys it sees
            s[h] += p[:, :C].sum(axis=0)           # accumulate per key j < C
    return s


# ----------------------------------------------------------------------------
# Top-K  [Summary, Methodology 1, Selection]
# ----------------------------------------------------------------------------

def _rank_order(s):
    """Indices ordered by score descending, ties to the lower index."""
    idx = np.arange(s.shape[0])
    return np.lexsort((idx, -s))


def topk_candidates(scores, k):
    """The k highest-scored positions (ties to the lower index), ascending.

    Comparisons happen in the dtype of ``scores`` (float32 scores are compared
    as float32, float64 as float64).
    """
    s = np.asarray(scores)
    if s.ndim != 1 or not 1 <= k <= s.shape[0]:
        raise ValueError("need 1 <= k <= len(scores)")
    if not np.all(np.isfinite(s)):
        raise ValueError("non-finite scores")
    return np.sort(_rank_order(s)[:k])


# ----------------------------------------------------------------------------
# Token2Chunk  [Summary, Methodology 2, Process / Outcome; Paper, Abstract]
# ----------------------------------------------------------------------------

def token2chunk(scores, cand, budget, return_spans=False):
    """Expand the candidates into chunks and fill the budget to exactly R.

    scores: [C] region scores; arithmetic of the chunk score runs in the dtype
            of ``scores`` (float32: one rounded add, one rounded divide).
    cand:   ascending candidate positions (the Top-K result).
    budget: R, kept tokens of the region, candidates included.

    Returns the R kept positions ascending (and, if asked, the accepted spans
    as (left endpoint, right endpoint) pairs in acceptance order).
    """
    s = np.asarray(scores)
    C = s.shape[0]
    cand = [int(c) for c in cand]
    K = len(cand)
    if any(cand[m] >= cand[m + 1] for m in range(K - 1)):
        raise ValueError("candidates must be strictly increasing")
    if not 1 <= budget <= C:
        raise ValueError("need 1 <= R <= C")
    if budget < K:
        kept = topk_candidates(s, budget)
        return (kept, []) if return_spans else kept

    ftype = s.dtype.type
    spans = []
    for m in range(K - 1):
        a, b = cand[m], cand[m + 1]
        gap = b - a - 1
        if gap == 0:
            continue                      # adjacent candidates leave nothing to add
        sigma = (s[a] + s[b]) / ftype(gap + 2)
        spans.append((sigma, a, b, gap))
    spans.sort(key=lambda t: (-t[0], t[1]))

    room = budget - K
    kept = np.zeros(C, dtype=bool)
    kept[cand] = True
    used = 0
    accepted = []
    for sigma, a, b, gap in spans:
        if used + gap > room:
            break                         # prefix greedy: stop at the first misfit
        used += gap
        kept[a + 1:b] = True
        accepted.append((a, b))

    need = budget - int(kept.sum())
    if need > 0:
        for j in _rank_order(s):
            if need == 0:
                break
            if not kept[j]:
                kept[j] = True
                need -= 1
    out = np.flatnonzero(kept)
    return (out, accepted) if return_spans else out


def select_retained(scores, top_k, budget, chunks=True):
    """Top-K then Token2Chunk on one unit's region scores; with chunks=False
    (the ablation) the kept set is the top-R set."""
    if not chunks:
        return topk_candidates(scores, budget)
    cand = topk_candidates(scores, top_k)
    return token2chunk(scores, cand, budget)


# ----------------------------------------------------------------------------
# Paged cache bookkeeping  [Summary, Methodology 3; Paper, Fig. 1 caption]
# ----------------------------------------------------------------------------

class PoolExhausted(RuntimeError):
    pass


class FifoPool:
    """Free list of block ids: allocation pops the front, freeing pushes the back."""

    def __init__(self, free_ids):
        self.q = deque(int(x) for x in free_ids)

    def __len__(self):
        return len(self.q)

    def pop(self, n):
        if n > len(self.q):
            raise PoolExhausted("not enough free blocks")
        return [self.q.popleft() for _ in range(n)]

    def push(self, ids):
        self.q.extend(int(x) for x in ids)

    def ids(self):
        return list(self.q)


def plan_compaction(table, lens, window, protect, budget, block_size, pool):
    """New block table rows and lengths for compressing every listed sequence.

    table: [S, MB] int block ids (entries past a sequence's end are ignored).
    lens:  [S] token counts, each >= W.
    pool:  FifoPool, updated in place (fresh ids popped for all sequences
           first, in call order; then the old trailing blocks pushed, in call
           order and by position).
    Returns (new_table [S, MB] with -1 past the new end, new_lens [S]).
    """
    table = np.asarray(table)
    S, MB = table.shape
    bs = block_size
    C = window - protect
    plans = []
    need = 0
    for b in range(S):
        L = int(lens[b])
        if L < window:
            raise ValueError("sequence shorter than the window")
        start = L - window
        f0 = start // bs
        p = start - f0 * bs
        n_new = ceil((p + budget + protect) / bs)
        plans.append((L, f0, n_new))
        need += n_new
    if need > len(pool):
        raise PoolExhausted("not enough free blocks")
    new_table = np.full((S, MB), -1, dtype=np.int64)
    new_lens = np.zeros(S, dtype=np.int64)
    for b, (L, f0, n_new) in enumerate(plans):
        new_table[b, :f0] = table[b, :f0]
        new_table[b, f0:f0 + n_new] = pool.pop(n_new)
        new_lens[b] = L - C + budget
    for b, (L, f0, n_new) in enumerate(plans):
        pool.push(table[b, f0:ceil(L / bs)])
    return new_table, new_lens


def _row(pool_arr, layer, kv, table_row, token, head, bs):
    return pool_arr[layer, kv, table_row[token // bs], head, token % bs]


def logical_tokens(pool_arr, table_row, length, layer, kv, head, block_size):
    """The rows [length, D] of one (layer, K/V, head) in logical token order."""
    return np.stack([_row(pool_arr, layer, kv, table_row, t, head, block_size)
                     for t in range(length)]) if length else np.zeros((0,) + pool_arr.shape[-1:], pool_arr.dtype)


def window_keys(pool_arr, table_row, length, window, layer, n_kv_heads, block_size):
    """Key rows of the trailing window, [W, Hkv, D]."""
    start = length - window
    return np.stack([
        np.stack([_row(pool_arr, layer, 0, table_row, start + i, h, block_size)
                  for h in range(n_kv_heads)])
        for i in range(window)])


def apply_compaction(pool_arr, table, lens, new_table, window, protect, budget,
                     block_size, retained):
    """Copy the kept rows into the fresh blocks; returns a new pool array.

    pool_arr: [Lyr, 2, NB, Hkv, bs, D] (K = 0, V = 1), copied value for value.
    retained: [S, Lyr, Hkv, R] window-local kept positions, ascending.
    New order of each (layer, K/V, head): the p tokens of the boundary block
    that precede the window, the R kept tokens, then the B protected tokens.
    """
    out = pool_arr.copy()
    Lyr, _, _, Hkv, bs, _ = pool_arr.shape
    assert bs == block_size
    S = len(lens)
    for b in range(S):
        L = int(lens[b])
        start = L - window
        f0 = start // bs
        base = f0 * bs                             # first token of the boundary block
        src_tokens = list(range(base, start))     # the boundary block's leading tokens
        for l in range(Lyr):
            for h in range(Hkv):
                kept = [start + int(j) for j in retained[b, l, h]]
                order = src_tokens + kept + list(range(L - protect, L))
                for kv in range(2):
                    for n, t in enumerate(order):
                        dst_blk = new_table[b, f0 + n // bs]
                        out[l, kv, dst_blk, h, n % bs] = _row(pool_arr, l, kv, table[b], t, h, bs)
    return out


# ----------------------------------------------------------------------------
# Around the step: the window's query states, and decode attention over the
# paged cache  [Summary, Methodology 1, Mechanism: the query states of all
# window tokens score the region; Paper, Abstract: the compressed cache is
# served through PagedAttention]
# ----------------------------------------------------------------------------

def window_queries(history, window):
    """Query states of a sequence's last W tokens, in token order.

    history: the query states [Lyr, Hq, D] of every token the sequence has
    produced so far, oldest first.  Returns [Lyr, W, Hq, D].  (Under the
    periodic schedule's watermark a window never reaches back into a region
    that was compacted, so its tokens are the last W produced.)
    """
    if len(history) < window:
        raise ValueError("fewer than W tokens produced")
    return np.stack(history[-window:], axis=1)


def decode_attention(q, pool_arr, table_row, length, layer, block_size):
    """Attention of one decode step's queries over a sequence's cached tokens.

    q: [Hq, D] query states of the sequence at `layer`.  The cache holds the
    sequence's `length` tokens in logical order through `table_row`.  Query
    head g reads KV head g // G: out[g] = sum_t softmax_t(q_g . k_t / sqrt(D))
    v_t.  Returns float64 [Hq, D].
    """
    q = np.asarray(q, dtype=np.float64)
    Hq, D = q.shape
    Hkv = pool_arr.shape[3]
    G = Hq // Hkv
    if length < 1:
        raise ValueError("empty sequence")
    out = np.zeros((Hq, D))
    for h in range(Hkv):
        k = logical_tokens(pool_arr, table_row, length, layer, 0, h, block_size).astype(np.float64)
        v = logical_tokens(pool_arr, table_row, length, layer, 1, h, block_size).astype(np.float64)
        for g in range(h * G, (h + 1) * G):
            x = (k @ q[g]) / np.sqrt(D)
            e = np.exp(x - x.max())
            out[g] = (e / e.sum()) @ v
    return out


# ----------------------------------------------------------------------------
# Periodic schedule  [Summary, Methodology 3, Periodic Compression Policy;
# Summary, Methodology intro: compression only of recently generated context]
# ----------------------------------------------------------------------------

def schedule_step(step, period, window, lens, watermarks, selected):
    """Sequences compressed at decode step `step`, ascending.

    Only at positive multiples of the period; among the caller's selected
    sequences, those whose trailing window holds only tokens that have not yet
    been through a compressed region (length - watermark >= W).  The caller
    moves a compressed sequence's watermark to new_length - B.
    """
    if step <= 0 or step % period:
        return []
    return [b for b in range(len(lens)) if selected[b] and lens[b] - watermarks[b] >= window]


# ----------------------------------------------------------------------------
# End to end
# ----------------------------------------------------------------------------

def compress(q_window, pool_arr, table, lens, window, protect, top_k, budget,
             block_size, free_ids, units=None, unidirectional=False, chunks=True):
    """Whole step on host arrays.

    q_window: [S, Lyr, W, Hq, D]; pool_arr: [Lyr, 2, NB, Hkv, bs, D].
    free_ids: the pool's free list, front first.
    units:    optional iterable of (b, l) pairs to score; other pairs are left
              unscored (used to sample large workloads).  Compaction needs
              every unit, so it runs only when ``units`` is None.
    unidirectional, chunks: the ablations (see the module header).
    Returns a dict with scores [S, Lyr, Hkv, C], cand [S, Lyr, Hkv, K],
    retained [S, Lyr, Hkv, R] (rows not scored hold -1), and when compacted:
    pool, table, lens, free_ids.
    """
    q_window = np.asarray(q_window)
    S, Lyr, W, Hq, D = q_window.shape
    assert W == window
    Hkv = pool_arr.shape[3]
    C = window - protect
    scores = np.full((S, Lyr, Hkv, C), np.nan)
    cand = np.full((S, Lyr, Hkv, top_k), -1, dtype=np.int64)
    retained = np.full((S, Lyr, Hkv, budget), -1, dtype=np.int64)
    todo = [(b, l) for b in range(S) for l in range(Lyr)] if units is None else list(units)
    for b, l in todo:
        k_win = window_keys(pool_arr, table[b], int(lens[b]), window, l, Hkv, block_size)
        s = window_scores(q_window[b, l], k_win, protect, unidirectional)
        scores[b, l] = s
        for h in range(Hkv):
            c = topk_candidates(s[h], top_k)
            cand[b, l, h] = c
            retained[b, l, h] = token2chunk(s[h], c, budget) if chunks else topk_candidates(s[h], budget)
    out = dict(scores=scores, cand=cand, retained=retained)
    if units is None:
        pool = FifoPool(free_ids)
        new_table, new_lens = plan_compaction(table, lens, window, protect, budget, block_size, pool)
        out["pool"] = apply_compaction(pool_arr, table, lens, new_table, window, protect,
                                       budget, block_size, retained)
        out["table"] = new_table
        out["lens"] = new_lens
        out["free_ids"] = pool.ids()
    return out
