"""Verification-guided KV selection (oracle; test infrastructure only).

Definitions followed
--------------------
* Vegas page, "Core claim" and "What carries the argument": the pre-softmax
  logits of the first draft token and the bonus token are combined across the
  query heads, and the k prefix positions with the largest combined score are
  kept for the next drafting phase.  The page only paraphrases its Eq. 3; we
  sum the two rows over the heads (a head mean is the same ranking divided by
  the positive constant 2H).
* Sparse Glimpse page, "Core claim": the sparse set keeps sink tokens, recent
  tokens and the top-ranked historical tokens, per head.  Here that is the
  per-KV-head mode: one set per KV head, scored over the query heads of its
  group.
* SSV page, "What carries the argument" / Figure 3 caption: NSA selects
  hardware-aligned blocks.  A block's score is the max of the position scores
  inside it (no formula is printed; max is the plainest reading).  The
  alternative aggregation is the block's log-sum-exp, log sum_p exp(sigma_p),
  a smooth max that also counts how many strong positions a block holds.

Selection rule (the pages are silent on these points; our readings):
1. sigma_p = sum over heads in the set of (l[h, row0, p] + l[h, row1, p]).
2. If L <= n_sink + K + n_recent every prefix position is kept.
3. Otherwise the pool is [n_sink, L - n_recent); the K pool positions with the
   largest sigma are kept, ties going to the smaller position; the sink
   [0, n_sink) and recent [L - n_recent, L) windows are always kept.
4. The output is ascending.

``scores_f32_pinned`` is the same score in float32 with the summation order
fixed (heads ascending, each pair summed first); the GPU selector must match
it bit for bit, so the top-k on the GPU's own logits can be compared exactly.

Scoring variants (rule 1 with other inputs; readings of ours):
* n collected rows instead of two: each head contributes the sum of its n rows'
  logits (in float32: t = l0, then t = t + l_c in slot order, then the head sum).
  All n_q rows is the all-row collection the Vegas page's Figure 6 prices.
* Softmax weights (Sparse Glimpse page, "Core claim" and its parameter list: the
  per-head attention weights of the last W = 16 verification queries are the
  importance signal): each head contributes, over its collected rows r, the
  weight exp(l[h, r, p] - lse[h, r]) of position p.  The page gives no formula for
  the aggregation; a plain sum over rows and over the set's heads is ours.
"""
from __future__ import annotations

import numpy as np


def set_heads(mode: str, Hq: int, Hkv: int, s: int):
    """Query heads whose logits score set s (s = 0 for 'shared', s = g otherwise)."""
    if mode == "shared":
        return list(range(Hq))
    G = Hq // Hkv
    return list(range(s * G, (s + 1) * G))


def n_sets(mode: str, Hkv: int) -> int:
    return 1 if mode == "shared" else Hkv


def scores_f64(logits: np.ndarray, b: int, L: int, heads) -> np.ndarray:
    """sigma_p in float64 for p < L (exact sum of float64 values, order irrelevant)."""
    x = np.asarray(logits[b, heads, :, :L], dtype=np.float64)
    return np.sum(x, axis=(0, 1))


def scores_f32_pinned(logits: np.ndarray, b: int, L: int, heads) -> np.ndarray:
    """sigma_p in float32, pinned order: acc = 0; for h ascending: acc = acc + t_h,
    t_h = l0 for one row, (l0 + l1) for two, (((l0 + l1) + l2) + ...) for more.

    Negative zero is mapped to positive zero so that the two compare and key
    identically.
    """
    x = np.asarray(logits[b, :, :, :L], dtype=np.float32)
    acc = np.zeros(L, dtype=np.float32)
    for h in heads:
        t = x[h, 0].copy()
        for c in range(1, x.shape[1]):
            t = (t + x[h, c]).astype(np.float32)
        acc = (acc + t).astype(np.float32)
    acc[acc == 0] = np.float32(0.0)
    return acc


def partial_scores_f32(logits: np.ndarray, b: int, L: int, Hq: int, Hkv: int) -> np.ndarray:
    """Per-KV-head partial scores [Hkv][L] in float32: row g is the pinned-order score
    of the G query heads of group g (acc = 0; acc = acc + (l0 + l1) over its heads).

    Selecting from these, the shared score is the pinned sum over g of the rows
    (grouped association), and a KV head's set scores by its own row, which is
    exactly its per-KV-head score on the logits.
    """
    G = Hq // Hkv
    return np.stack([scores_f32_pinned(logits, b, L, range(g * G, (g + 1) * G)) for g in range(Hkv)])


def scores_weights_f64(logits: np.ndarray, lse: np.ndarray, rows, b: int, L: int, heads) -> np.ndarray:
    """Softmax-weight score in float64: sum over heads h and slots c of
    exp(l[b, h, c, p] - lse[b, rows[c], h]) for p < L.

    logits [B][Hq][n_rows][ld] (slot c = verifier row rows[c]); lse [B][n_q][Hq],
    natural log, over every position the row sees.
    """
    x = np.asarray(logits[b, :, :, :L], dtype=np.float64)
    acc = np.zeros(L)
    for h in heads:
        for c, r in enumerate(rows):
            acc += np.exp(x[h, c] - float(lse[b, r, h]))
    return acc


def topk_tokens(sigma: np.ndarray, L: int, top_k: int, n_sink: int, n_recent: int) -> np.ndarray:
    """Selection rule for token sets; returns ascending int64 positions."""
    if L <= n_sink + top_k + n_recent:
        return np.arange(L, dtype=np.int64)
    lo, hi = n_sink, L - n_recent
    pool = np.arange(lo, hi, dtype=np.int64)
    order = np.lexsort((pool, -sigma[lo:hi]))   # sigma descending, position ascending
    chosen = pool[order[:top_k]]
    return np.sort(np.concatenate([np.arange(0, n_sink), chosen, np.arange(hi, L)]).astype(np.int64))


def block_window(L: int, bs: int, n_sink: int, n_recent: int):
    """(n_blocks, first pool block, end of pool) for block selection.

    Blocks that hold any sink position are always kept; so are blocks that
    overlap [L - n_recent, L).
    """
    nb = (L + bs - 1) // bs
    sb = (n_sink + bs - 1) // bs
    rb = (L - n_recent) // bs if n_recent > 0 else nb
    return nb, sb, rb


def block_scores(sigma: np.ndarray, L: int, bs: int) -> np.ndarray:
    """beta_c = max of sigma over the prefix positions inside block c."""
    nb = (L + bs - 1) // bs
    return np.array([np.max(sigma[c * bs:min(L, (c + 1) * bs)]) for c in range(nb)],
                    dtype=sigma.dtype)


def block_scores_lse(sigma: np.ndarray, L: int, bs: int) -> np.ndarray:
    """beta_c = log sum over the prefix positions p of block c of exp(sigma_p), in
    float64 (shifted by the block's max, which leaves the value unchanged)."""
    nb = (L + bs - 1) // bs
    out = np.empty(nb)
    for c in range(nb):
        x = np.asarray(sigma[c * bs:min(L, (c + 1) * bs)], dtype=np.float64)
        m = np.max(x)
        out[c] = m + np.log(np.sum(np.exp(x - m)))
    return out


def topk_blocks(sigma: np.ndarray, L: int, top_k: int, n_sink: int, n_recent: int,
                bs: int, agg: str = "max") -> np.ndarray:
    """Block selection rule; returns ascending int64 block ids.  agg: "max" or "lse"."""
    nb, sb, rb = block_window(L, bs, n_sink, n_recent)
    if sb >= rb or nb <= sb + top_k + (nb - rb):
        return np.arange(nb, dtype=np.int64)
    beta = block_scores(sigma, L, bs) if agg == "max" else block_scores_lse(sigma, L, bs)
    pool = np.arange(sb, rb, dtype=np.int64)
    order = np.lexsort((pool, -beta[sb:rb]))
    chosen = pool[order[:top_k]]
    return np.sort(np.concatenate([np.arange(0, sb), chosen, np.arange(rb, nb)]).astype(np.int64))


def select(logits: np.ndarray, prefix_len: np.ndarray, Hkv: int, mode: str, top_k: int,
           n_sink: int, n_recent: int, block_size: int = 0, precision: str = "f64",
           score_kind: str = "logits", lse: np.ndarray = None, rows=None, block_agg: str = "max"):
    """Run the selector for every (sequence, set).

    logits: [B][Hq][n_rows][ld] (the collected rows; two for Collect-2-Query).
    score_kind "weights" scores by softmax weights (needs lse [B][n_q][Hq] and the
    verifier row of each slot, rows).  block_agg "max" or "lse" aggregates a block's
    position scores in block mode.  Returns a list over b of lists over sets of
    ascending int64 arrays (positions, or block ids in 'block' mode, where sets
    are per KV head).
    """
    B, Hq = logits.shape[0], logits.shape[1]
    if score_kind == "weights":
        def score(lg, b, L, heads):
            return scores_weights_f64(lg, lse, rows, b, L, heads)
    else:
        score = scores_f64 if precision == "f64" else scores_f32_pinned
    res = []
    for b in range(B):
        L = int(prefix_len[b])
        per = []
        smode = "per_kv_head" if mode == "block" else mode
        for s in range(n_sets(smode, Hkv)):
            sig = score(logits, b, L, set_heads(smode, Hq, Hkv, s))
            if mode == "block":
                per.append(topk_blocks(sig, L, top_k, n_sink, n_recent, block_size, block_agg))
            else:
                per.append(topk_tokens(sig, L, top_k, n_sink, n_recent))
        res.append(per)
    return res


def pack(res, cap: int):
    """List-of-lists result -> (indices int32 [B][n_sets][cap] padded with -1, counts [B][n_sets])."""
    B, S = len(res), len(res[0])
    idx = np.full((B, S, cap), -1, dtype=np.int32)
    cnt = np.zeros((B, S), dtype=np.int32)
    for b in range(B):
        for s in range(S):
            a = res[b][s]
            idx[b, s, :a.size] = a
            cnt[b, s] = a.size
    return idx, cnt


def to_physical(positions: np.ndarray, block_table: np.ndarray, b: int, page_size: int) -> np.ndarray:
    """Physical cache slots of sequence b's logical positions: the paged layout puts
    position p in page block_table[b][p // P] at slot p % P, i.e. slot page * P + p % P
    (the hand-off of a selection to the draft as physical rows)."""
    p = np.asarray(positions, dtype=np.int64)
    return (block_table[b][p // page_size].astype(np.int64) * page_size + p % page_size).astype(np.int64)
