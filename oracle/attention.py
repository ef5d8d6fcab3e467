"""Attention over the de-paged cache, in fp64 (oracle; test infrastructure only).

Definition (Tutorial §2, "Attention(Q, K, V) = softmax(QK^T / sqrt(d)) V";
Lecture 10 "KV Cache 原理": at a decode step the new token's query is scored
against every cached key and the scores weight a sum of every cached value):

    for query row q, keys K[0..lam), values V[0..lam), scale sigma:
        s_t  = sigma * sum_k q[k] * K[t, k]
        out  = sum_t exp(s_t) V[t] / sum_t exp(s_t)
        lse  = log sum_t exp(s_t)

The row maximum m is subtracted inside exp (exp(s_t - m) / sum exp(s_u - m) is
the same softmax); it only keeps the fp64 exponentials finite.

GQA (Lecture 10 "Grouped Query Attention"; Tutorial §3): query heads are split
into groups that share one K/V head, n_kv_heads = n_heads / group_size.  The
pages give no index rule; heads are taken in contiguous groups, so query head h
reads KV head h // (n_heads / n_kv_heads).

Verify (Guide §4.2, Lecture 10 "Speculative Decoding"): the target model scores
the last token and the K draft tokens in ONE forward.  With seq_len L counting
those nq = K + 1 positions, query position i (0 <= i < nq) sits at absolute
position L - nq + i and, being causal, sees tokens t <= L - nq + i, that is the
first lam_i = L - nq + 1 + i tokens.  Decode is nq = 1, lam = L.

Sliding window (in-depth guide §2.3, "稀疏注意力与窗口化的工程取舍": each token attends
only to the most recent W tokens).  Reading taken: the W tokens end at and include the
row's own position p, so a row sees tokens max(0, p - W + 1) .. p; W = 0 means no window
(the whole causal prefix).

Multi-query rows (guide §3.3 speculative trees; §4.1 chunked prefill): the last nq
tokens of a sequence are query positions, already in the cache.  Chunked prefill is the
causal case above with nq up to a few hundred.  A speculative tree puts nq candidate
tokens in the cache in tree order (a parent before its children); candidate i then sees
every context token t < L - nq and the candidate j (position L - nq + j) only if j is i
itself or one of its ancestors.  Reading taken: the tree arrives as a visibility mask
mask[i][j] over the nq candidates (1 = visible), so any mask, the causal one included,
is accepted.

Context split (not on the pages; stated by the benchmark spec): the tokens visible to a row
are cut into partitions, attention is taken over each (o_p, lse_p), and the
partials are recombined with the log-sum-exp identity

    M = max_p lse_p,  w_p = exp(lse_p - M),
    out = sum_p w_p o_p / sum_p w_p,  lse = M + log sum_p w_p,

which is exact because exp(lse_p) is partition p's softmax denominator.
A row that sees no token has out = 0 and lse = -inf.
"""

import numpy as np

from . import paging, storage


def attend(q_rows, K, V, sigma, limits, starts=None):
    """fp64 attention of each row of ``q_rows`` ([R, d]) over rows
    [starts[r], limits[r]) of K and V ([L, d]) (starts default to 0).
    Returns (out [R, d], lse [R])."""
    q_rows = np.asarray(q_rows, dtype=np.float64)
    R, d = q_rows.shape
    out = np.zeros((R, d), dtype=np.float64)
    lse = np.full((R,), -np.inf, dtype=np.float64)
    for r in range(R):
        lam = int(limits[r])
        lo = 0 if starts is None else max(0, int(starts[r]))
        if lam <= lo:
            continue
        s = sigma * (K[lo:lam] @ q_rows[r])
        m = s.max()
        e = np.exp(s - m)
        l = e.sum()
        out[r] = (e @ V[lo:lam]) / l
        lse[r] = m + np.log(l)
    return out, lse


def row_limits(seq_len, num_q_pos):
    """Visible-token count of each query position (causal verify rows)."""
    return [max(0, seq_len - num_q_pos + 1 + i) for i in range(num_q_pos)]


def row_starts(seq_len, num_q_pos, window):
    """First visible token of each query position: with a sliding window of W > 0 tokens
    the row at position p starts at max(0, p - W + 1); with W = 0 at token 0."""
    if window <= 0:
        return [0] * num_q_pos
    return [max(0, lam - window) for lam in row_limits(seq_len, num_q_pos)]


def attend_indices(q_rows, K, V, sigma, index_lists):
    """fp64 attention of each row over the rows index_lists[r] of K and V."""
    q_rows = np.asarray(q_rows, dtype=np.float64)
    R, d = q_rows.shape
    out = np.zeros((R, d), dtype=np.float64)
    lse = np.full((R,), -np.inf, dtype=np.float64)
    for r in range(R):
        idx = np.asarray(index_lists[r], dtype=np.int64)
        if idx.size == 0:
            continue
        s = sigma * (K[idx] @ q_rows[r])
        m = s.max()
        e = np.exp(s - m)
        l = e.sum()
        out[r] = (e @ V[idx]) / l
        lse[r] = m + np.log(l)
    return out, lse


def tree_visible(seq_len, num_q_pos, i, mask_row):
    """Tokens query position i sees under a candidate mask: all context tokens
    t < seq_len - nq, then candidate j at seq_len - nq + j where mask_row[j] is set
    (candidates before position 0 of the sequence do not exist)."""
    base = seq_len - num_q_pos
    ctx = list(range(max(0, base)))
    return ctx + [base + j for j in range(num_q_pos) if mask_row[j] and base + j >= 0]


def _group_rows(q_dec, b, g, G, num_q_pos):
    """Rows (i, head) of sequence b that read KV head g, in (i, head) order."""
    rows, idx = [], []
    for i in range(num_q_pos):
        for hg in range(G):
            h = g * G + hg
            rows.append(q_dec[b, i, h])
            idx.append((i, h))
    return np.stack(rows), idx


def paged_attention(q, q_kind, k_cache, v_cache, kv_kind, block_tables, seq_lens, sigma,
                    num_q_pos=1, k_scale=None, v_scale=None, pairs=None, fast=True, window=0,
                    tree_mask=None):
    """Attention of every query row against its sequence's paged cache.

    q: [B, nq, Hq, d] stored as ``q_kind``; caches in the project format (see
    ``paging``).  Returns (out [B, nq, Hq, d], lse [B, nq, Hq]) in fp64.  With
    ``pairs`` (a list of (b, g)) only those sequence/KV-head pairs are computed and
    every other entry is NaN.  ``sigma`` is used as given (pass the fp32 value the
    kernel receives, widened).  ``window`` > 0: sliding-window attention over the
    ``window`` most recent tokens of each row (``row_starts``).  ``tree_mask``
    ([B, nq, nq] booleans, or None for causal rows): candidate visibility
    (``tree_visible``); it is not combined with a window.
    """
    qd = storage.decode(q, q_kind)
    B, nq, Hq, d = qd.shape
    assert nq == num_q_pos
    Hkv = k_cache.shape[1]
    G = Hq // Hkv
    out = np.full((B, nq, Hq, d), np.nan)
    lse = np.full((B, nq, Hq), np.nan)
    if pairs is None:
        pairs = [(b, g) for b in range(B) for g in range(Hkv)]
    dep = paging.depage_fast if fast else paging.depage
    for b, g in pairs:
        L = int(seq_lens[b])
        K, V = dep(k_cache, v_cache, kv_kind, block_tables[b], L, g, k_scale, v_scale)
        rows, idx = _group_rows(qd, b, g, G, nq)
        if tree_mask is None:
            lim = row_limits(L, nq)
            lo = row_starts(L, nq, window)
            o, ls = attend(rows, K, V, sigma, [lim[i] for i, _ in idx], [lo[i] for i, _ in idx])
        else:
            vis = [tree_visible(L, nq, i, tree_mask[b][i]) for i in range(nq)]
            o, ls = attend_indices(rows, K, V, sigma, [vis[i] for i, _ in idx])
        for r, (i, h) in enumerate(idx):
            out[b, i, h] = o[r]
            lse[b, i, h] = ls[r]
    return out, lse


def partitions_used(seq_len, partition_tokens, max_partitions):
    """Number of partitions a sequence of ``seq_len`` tokens occupies: one per
    ``partition_tokens`` tokens, at most ``max_partitions`` (the last one then also
    takes every remaining token)."""
    if seq_len <= 0:
        return 0
    return min(-(-seq_len // partition_tokens), max_partitions)


def partition_range(seq_len, p, partition_tokens, max_partitions):
    """Token range [lo, hi) of partition p."""
    n = partitions_used(seq_len, partition_tokens, max_partitions)
    lo = p * partition_tokens
    hi = seq_len if p == n - 1 else min(seq_len, (p + 1) * partition_tokens)
    return lo, hi


def paged_attention_partitions(q, q_kind, k_cache, v_cache, kv_kind, block_tables, seq_lens,
                               sigma, partition_tokens, max_partitions, num_q_pos=1,
                               k_scale=None, v_scale=None, pairs=None):
    """Per-partition partial attention (o_p, lse_p).

    Returns (o [B, nq, Hq, P, d], lse [B, nq, Hq, P]) with P = max_partitions;
    partition p of a row attends over the tokens of [lo_p, hi_p) that the row may
    see.  Entries of partitions a sequence does not occupy are NaN.
    """
    qd = storage.decode(q, q_kind)
    B, nq, Hq, d = qd.shape
    Hkv = k_cache.shape[1]
    G = Hq // Hkv
    P = max_partitions
    o = np.full((B, nq, Hq, P, d), np.nan)
    ls = np.full((B, nq, Hq, P), np.nan)
    if pairs is None:
        pairs = [(b, g) for b in range(B) for g in range(Hkv)]
    for b, g in pairs:
        L = int(seq_lens[b])
        K, V = paging.depage_fast(k_cache, v_cache, kv_kind, block_tables[b], L, g,
                                  k_scale, v_scale)
        rows, idx = _group_rows(qd, b, g, G, nq)
        lim = row_limits(L, nq)
        for p in range(partitions_used(L, partition_tokens, max_partitions)):
            lo, hi = partition_range(L, p, partition_tokens, max_partitions)
            # rows see tokens [lo, min(hi, lam)); shift K/V so the window starts at 0
            lims = [max(0, min(hi, lim[i]) - lo) for i, _ in idx]
            op, lp = attend(rows, K[lo:hi], V[lo:hi], sigma, lims)
            for r, (i, h) in enumerate(idx):
                o[b, i, h, p] = op[r]
                ls[b, i, h, p] = lp[r]
    return o, ls


def lse_merge(o_parts, lse_parts, n_parts=None):
    """Log-sum-exp recombination of partial attention results.

    o_parts [..., P, d], lse_parts [..., P]; ``n_parts`` (broadcast against the
    leading dims) limits each row to its first n partitions.  Partitions with
    lse = -inf carry no weight.  Returns (out [..., d], lse [...]).
    """
    o_parts = np.asarray(o_parts, dtype=np.float64)
    lse_parts = np.asarray(lse_parts, dtype=np.float64)
    lead = lse_parts.shape[:-1]
    P = lse_parts.shape[-1]
    if n_parts is None:
        n_parts = np.full(lead, P)
    n_parts = np.broadcast_to(np.asarray(n_parts), lead)
    out = np.zeros(lead + (o_parts.shape[-1],))
    lse = np.full(lead, -np.inf)
    for ix in np.ndindex(*lead):
        n = int(n_parts[ix])
        lp = lse_parts[ix][:n]
        live = np.isfinite(lp)
        if not live.any():
            continue
        M = lp[live].max()
        w = np.exp(lp[live] - M)
        out[ix] = (w[:, None] * o_parts[ix][:n][live]).sum(0) / w.sum()
        lse[ix] = M + np.log(w.sum())
    return out, lse
