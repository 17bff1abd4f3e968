"""Dense verify attention and sparse draft attention, fp64 (oracle; test infrastructure only).

Definitions followed
--------------------
* Vegas page, "The pith" and "Core claim": verification runs full attention
  for all verifier tokens over the whole KV cache, and the pre-softmax logits
  of two rows (the first draft token and the bonus token) are exposed; the
  draft phase attends only to the selected prefix positions.
* Vegas page, Figure 6 caption: "Collect-2-Query" writes the logits of those
  two query rows only.
* SSV page, section 4.2 (exact merged-schedule variant) and the Figure 6 text:
  each verifier row keeps its own selection and its own causal boundary at its
  absolute position.

Readings taken where the pages are silent (listed in the design notes):
scale = 1/sqrt(d) is applied before the logits are exposed; query head h uses
KV head h // (Hq/Hkv); verifier row i sits at cache position L_b + i and sees
the prefix plus verifier slots j <= i (or the slots its tree mask names).

Everything is computed in float64 from the exact bf16 inputs, by the plain
definition: s = scale * q.k, softmax over the visible set, O = sum p * v,
lse = m + log(sum exp(s - m)).
"""
from __future__ import annotations

from typing import Optional, Sequence

import numpy as np


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns -> float64 (exact: bf16 is the top half of a float32)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def paged_rows(cache_bits: np.ndarray, block_table: np.ndarray, b: int, g: int,
               positions: np.ndarray, page_size: int) -> np.ndarray:
    """Rows of KV head g at logical positions of sequence b, as float64 [n][d].

    Logical position p lives in physical page block_table[b][p // P] at slot
    p % P (paged KV cache as used by the vLLM PagedAttention backend the Vegas
    page names).
    """
    positions = np.asarray(positions, dtype=np.int64)
    pages = block_table[b][positions // page_size].astype(np.int64)
    return bf16_to_f64(cache_bits[pages, g, positions % page_size, :])


def _softmax_stats(s: np.ndarray, visible: np.ndarray):
    """Masked softmax over the last axis.  Returns (P, lse) with P zero where hidden."""
    s = np.where(visible, s, -np.inf)
    m = np.max(s, axis=-1, keepdims=True)
    w = np.where(visible, np.exp(s - m), 0.0)
    l = np.sum(w, axis=-1, keepdims=True)
    return w / l, (m + np.log(l))[..., 0]


def verify_visibility(prefix_len: int, n_q: int, tail_mask: Optional[Sequence[int]]) -> np.ndarray:
    """[n_q][prefix_len + n_q] bool: row i sees the prefix and verifier slot j if allowed.

    Chain default: slot j is visible to row i iff j <= i.  With a tree mask,
    slot j is visible iff bit j of tail_mask[i] is set.
    """
    L = int(prefix_len)
    vis = np.zeros((n_q, L + n_q), dtype=bool)
    vis[:, :L] = True
    for i in range(n_q):
        for j in range(n_q):
            if tail_mask is None:
                ok = j <= i
            else:
                ok = (int(tail_mask[i]) >> j) & 1 == 1
            vis[i, L + j] = ok
    return vis


def verify_attn(q_bits: np.ndarray, k_bits: np.ndarray, v_bits: np.ndarray,
                block_table: np.ndarray, prefix_len: np.ndarray, page_size: int,
                scale: float, tree_mask: Optional[np.ndarray] = None,
                collect_rows: Sequence[int] = None, logits_ld: Optional[int] = None,
                return_weights: bool = False):
    """Dense verify attention over the full paged cache, plus collected logit rows.

    q_bits: bf16 [B][n_q][Hq][d]; k_bits/v_bits: bf16 [pages][Hkv][P][d].
    Returns (out [B][n_q][Hq][d], logits [B][Hq][n_c][ld], lse [B][n_q][Hq]) in
    float64; slot c of logits holds scale*q.k of row collect_rows[c] (default
    the two rows 0 and n_q - 1, the Vegas page's Collect-2-Query pair) for
    prefix columns p < prefix_len[b], NaN elsewhere.  With return_weights the
    softmax weights [b][g] -> [n_q][G][L_b+n_q] are returned as a fourth item.
    """
    B, n_q, Hq, d = q_bits.shape
    Hkv = k_bits.shape[1]
    G = Hq // Hkv
    if collect_rows is None:
        collect_rows = (0, n_q - 1)
    Lmax = int(np.max(prefix_len)) if B else 0
    ld = Lmax if logits_ld is None else logits_ld
    out = np.zeros((B, n_q, Hq, d))
    lse = np.zeros((B, n_q, Hq))
    logits = np.full((B, Hq, len(collect_rows), ld), np.nan)
    weights = {}
    q = bf16_to_f64(q_bits)
    for b in range(B):
        L = int(prefix_len[b])
        pos = np.arange(L + n_q)
        vis = verify_visibility(L, n_q, None if tree_mask is None else tree_mask[b])
        for g in range(Hkv):
            K = paged_rows(k_bits, block_table, b, g, pos, page_size)
            V = paged_rows(v_bits, block_table, b, g, pos, page_size)
            Qg = q[b, :, g * G:(g + 1) * G, :]                 # [n_q][G][d]
            S = scale * np.einsum("igd,pd->igp", Qg, K)         # [n_q][G][L+n_q]
            P, row_lse = _softmax_stats(S, vis[:, None, :])
            out[b, :, g * G:(g + 1) * G, :] = np.einsum("igp,pd->igd", P, V)
            lse[b, :, g * G:(g + 1) * G] = row_lse
            for c, r in enumerate(collect_rows):
                logits[b, g * G:(g + 1) * G, c, :L] = S[r, :, :L]
            if return_weights:
                weights[(b, g)] = P
    if return_weights:
        return out, logits, lse, weights
    return out, logits, lse


def sparse_visible_positions(mode: str, indices: np.ndarray, counts: np.ndarray, b: int,
                             row: int, g: int, page_size: int, tail_begin: int) -> np.ndarray:
    """Selected prefix positions that (row, KV head g) of sequence b attends to.

    shared:      indices [B][1][cap]        one list per sequence (Vegas)
    per_kv_head: indices [B][Hkv][cap]      one list per KV head (Sparse Glimpse)
    block:       indices [B][n_q][Hkv][cap] block ids per row (SSV / NSA); a
                 block c covers [c*P, c*P + P) clipped to the prefix.
    """
    if mode == "shared":
        n = int(counts[b, 0])
        return np.asarray(indices[b, 0, :n], dtype=np.int64)
    if mode == "per_kv_head":
        n = int(counts[b, g])
        return np.asarray(indices[b, g, :n], dtype=np.int64)
    if mode == "block":
        n = int(counts[b, row, g])
        blocks = np.asarray(indices[b, row, g, :n], dtype=np.int64)
        if n == 0:
            return np.zeros(0, dtype=np.int64)
        toks = (blocks[:, None] * page_size + np.arange(page_size)[None, :]).reshape(-1)
        return toks[toks < tail_begin]
    raise ValueError(mode)


def sparse_attn(q_bits: np.ndarray, k_bits: np.ndarray, v_bits: np.ndarray,
                block_table: np.ndarray, page_size: int, mode: str,
                indices: np.ndarray, counts: np.ndarray, tail_begin: np.ndarray,
                tail_len: np.ndarray, scale: float,
                tail_mask: Optional[np.ndarray] = None):
    """Attention of each query row over its selected positions plus the tail.

    Row i of sequence b sees the selected prefix positions (see
    :func:`sparse_visible_positions`) and the tail slots tail_begin[b] + j,
    j < tail_len[b], whose bit j is set in tail_mask[b][i] (all of them when
    tail_mask is None).  Returns (out [B][n_q][Hq][d], lse [B][n_q][Hq]) in
    float64; a row with nothing visible gets out = 0 and lse = -inf.
    """
    B, n_q, Hq, d = q_bits.shape
    Hkv = k_bits.shape[1]
    G = Hq // Hkv
    out = np.zeros((B, n_q, Hq, d))
    lse = np.full((B, n_q, Hq), -np.inf)
    q = bf16_to_f64(q_bits)
    for b in range(B):
        tb, tl = int(tail_begin[b]), int(tail_len[b])
        for g in range(Hkv):
            for i in range(n_q):
                sel = sparse_visible_positions(mode, indices, counts, b, i, g, page_size, tb)
                tail = [tb + j for j in range(tl)
                        if tail_mask is None or ((int(tail_mask[b][i]) >> j) & 1)]
                pos = np.concatenate([sel, np.asarray(tail, dtype=np.int64)])
                if pos.size == 0:
                    continue
                K = paged_rows(k_bits, block_table, b, g, pos, page_size)
                V = paged_rows(v_bits, block_table, b, g, pos, page_size)
                Qi = q[b, i, g * G:(g + 1) * G, :]               # [G][d]
                S = scale * (Qi @ K.T)                           # [G][n]
                P, row_lse = _softmax_stats(S, np.ones_like(S, dtype=bool))
                out[b, i, g * G:(g + 1) * G, :] = P @ V
                lse[b, i, g * G:(g + 1) * G] = row_lse
    return out, lse


def attention_one(q_row: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float):
    """Plain softmax attention of one float64 query over float64 K/V rows.

    Returns (o [d], p [n], lse).  Used for sampled checks at full size, where
    the caller gathers the visible rows itself.
    """
    s = scale * (K @ q_row)
    m = np.max(s)
    w = np.exp(s - m)
    l = np.sum(w)
    p = w / l
    return p @ V, p, m + np.log(l)
