"""NSA branches for sparse speculative verification (oracle; test infrastructure only).

Definitions followed
--------------------
* SSV page, Figure 3 overview: NSA attention runs three branches for every query,
  token compression, token selection and a sliding window, and the verifier rows of a
  draft tree go through all three.  The selection branch is the block-sparse
  attention of ``oracle.attention.sparse_attn`` (mode "block").
* SSV page, Figure 10 caption: the grouped-query kernel runs in one of three modes,
  no grouping, exact or approximate.  Exact keeps every row's own block set while
  the group loads the union once (section 4.2, exact merged schedule); approximate
  lets every row of the group attend to the whole union.
* SSV page, Figure 3 text: reuse layers take the index of the nearest preceding
  refresh layer and skip index derivation; that changes which block lists a layer
  reads, not what the branches compute.

The pages name the branches but print no formula for them.  Readings taken (listed
with the others in the design notes):
* compression: block i of a sequence covers positions [i*s, i*s + l) and exists once
  the whole block lies in the prefix (i*s + l <= L).  Its key (value) is the mean of
  the block's l keys (values).  NSA learns this map (an MLP over the block); with no
  trained weights the mean is the plain parameter-free instance.  The compressed
  cache has the cache's type: the mean is rounded to bfloat16, to nearest, ties to
  even.
* the compression branch of a row attends to every compressed block of its
  sequence's prefix (the draft tokens are not compressed yet);
* the sliding window of a row is the last ``window`` prefix positions plus the
  draft (tail) tokens the row sees;
* the selection branch of a row is its blocks (exact) or the union of its group's
  blocks (approximate), clipped to the prefix, plus the tail tokens the row sees;
* gating: out = g_cmp * o_cmp + g_slc * o_slc + g_win * o_win with the caller's
  per-(row, head) gates; a branch that sees nothing contributes zero and reports
  lse = -inf.

All arithmetic is float64 on the exact bf16 inputs.
"""
from __future__ import annotations

from typing import Optional

import numpy as np

from .attention import bf16_to_f64, paged_rows, sparse_visible_positions


def round_bf16(x: np.ndarray) -> np.ndarray:
    """float64 -> bfloat16 bit patterns, rounding to nearest with ties to even, directly
    from the float64 value (8 significant bits).  Zero stays zero; inputs are finite
    and inside bf16's normal range."""
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)                      # x = m * 2**e, 0.5 <= |m| < 1
    r = np.ldexp(np.rint(np.ldexp(m, 8)), e - 8)   # 8 significant bits, ties to even
    bits = (r.astype(np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    return bits


def n_compressed(prefix_len: int, l: int, s: int) -> int:
    """Compressed blocks that lie entirely in a prefix of prefix_len positions."""
    return 0 if prefix_len < l else (prefix_len - l) // s + 1


def compress(k_bits: np.ndarray, v_bits: np.ndarray, block_table: np.ndarray, prefix_len: np.ndarray,
             page_size: int, l: int, s: int, max_cmp: Optional[int] = None):
    """Compressed K and V of every sequence and KV head.

    Returns (kc, vc) as bf16 bits [B][Hkv][max_cmp][d]; row i of (b, g) is the mean
    of positions [i*s, i*s + l) for i < n_compressed(prefix_len[b], l, s), rounded to
    bf16; rows past that are zero.
    """
    B = block_table.shape[0]
    Hkv, d = k_bits.shape[1], k_bits.shape[3]
    counts = [n_compressed(int(prefix_len[b]), l, s) for b in range(B)]
    M = max(counts + [1]) if max_cmp is None else max_cmp
    kc = np.zeros((B, Hkv, M, d), dtype=np.uint16)
    vc = np.zeros((B, Hkv, M, d), dtype=np.uint16)
    for b in range(B):
        n = counts[b]
        if n == 0:
            continue
        pos = np.arange(n * s - s + l)
        for g in range(Hkv):
            K = paged_rows(k_bits, block_table, b, g, pos, page_size)
            V = paged_rows(v_bits, block_table, b, g, pos, page_size)
            for i in range(n):
                kc[b, g, i] = round_bf16(K[i * s:i * s + l].mean(axis=0))
                vc[b, g, i] = round_bf16(V[i * s:i * s + l].mean(axis=0))
    return kc, vc


def _attend(Q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float):
    """Softmax attention of the rows of Q [G][d] over K/V [n][d]: (o [G][d], lse [G])."""
    if K.shape[0] == 0:
        return np.zeros((Q.shape[0], V.shape[1])), np.full(Q.shape[0], -np.inf)
    S = scale * (Q @ K.T)
    m = S.max(axis=1, keepdims=True)
    w = np.exp(S - m)
    z = w.sum(axis=1, keepdims=True)
    return (w / z) @ V, (m + np.log(z))[:, 0]


def union_sets(indices: np.ndarray, counts: np.ndarray):
    """Approximate grouping: every row of (b, g) gets the union of the rows' block ids.

    indices [B][n_q][Hkv][cap] -> (indices [B][n_q][Hkv][cap_u], counts), ascending.
    """
    B, n_q, Hkv, _ = indices.shape
    unions = [[np.unique(np.concatenate([indices[b, i, g, :counts[b, i, g]] for i in range(n_q)]))
               for g in range(Hkv)] for b in range(B)]
    cap_u = max([u.size for r in unions for u in r] + [1])
    out = np.full((B, n_q, Hkv, cap_u), -1, dtype=np.int32)
    cnt = np.zeros((B, n_q, Hkv), dtype=np.int32)
    for b in range(B):
        for g in range(Hkv):
            u = unions[b][g]
            out[b, :, g, :u.size] = u
            cnt[b, :, g] = u.size
    return out, cnt


def nsa_attn(q_bits: np.ndarray, k_bits: np.ndarray, v_bits: np.ndarray, block_table: np.ndarray,
             page_size: int, kc_bits: np.ndarray, vc_bits: np.ndarray, l: int, s: int,
             indices: np.ndarray, counts: np.ndarray, tail_begin: np.ndarray, tail_len: np.ndarray,
             window: int, gates: np.ndarray, scale: float, tail_mask: Optional[np.ndarray] = None,
             group: str = "exact"):
    """Gated three-branch NSA attention of the verifier rows.

    q_bits bf16 [B][n_q][Hq][d]; kc/vc bf16 [B][Hkv][M][d] (``compress``); block lists
    indices [B][n_q][Hkv][cap] / counts [B][n_q][Hkv] (block = page); tail_begin[b] =
    prefix length; row i sees tail slot j < tail_len[b] iff bit j of tail_mask[b][i]
    (all of them when tail_mask is None); gates fp [B][n_q][Hq][3] in the order
    (compression, selection, window).  group "exact" or "approximate".
    Returns (out [B][n_q][Hq][d], lse [B][n_q][Hq][3]) in float64.
    """
    B, n_q, Hq, d = q_bits.shape
    Hkv = k_bits.shape[1]
    G = Hq // Hkv
    if group == "approximate":
        indices, counts = union_sets(indices, counts)
    elif group != "exact":
        raise ValueError(group)
    q = bf16_to_f64(q_bits)
    kc = bf16_to_f64(kc_bits)
    vc = bf16_to_f64(vc_bits)
    gates = np.asarray(gates, dtype=np.float64)
    out = np.zeros((B, n_q, Hq, d))
    lse = np.full((B, n_q, Hq, 3), -np.inf)
    for b in range(B):
        tb, tl = int(tail_begin[b]), int(tail_len[b])
        nc = n_compressed(tb, l, s)
        for g in range(Hkv):
            for i in range(n_q):
                tail = np.array([tb + j for j in range(tl)
                                 if tail_mask is None or ((int(tail_mask[b][i]) >> j) & 1)], dtype=np.int64)
                Qi = q[b, i, g * G:(g + 1) * G, :]
                # compression branch
                o_c, l_c = _attend(Qi, kc[b, g, :nc], vc[b, g, :nc], scale)
                # selection branch
                sel = sparse_visible_positions("block", indices, counts, b, i, g, page_size, tb)
                pos = np.concatenate([sel, tail])
                o_s, l_s = _attend(Qi, paged_rows(k_bits, block_table, b, g, pos, page_size),
                                   paged_rows(v_bits, block_table, b, g, pos, page_size), scale)
                # sliding window branch
                pos = np.concatenate([np.arange(max(0, tb - window), tb, dtype=np.int64), tail])
                o_w, l_w = _attend(Qi, paged_rows(k_bits, block_table, b, g, pos, page_size),
                                   paged_rows(v_bits, block_table, b, g, pos, page_size), scale)
                gt = gates[b, i, g * G:(g + 1) * G, :]                      # [G][3]
                out[b, i, g * G:(g + 1) * G, :] = (gt[:, 0:1] * o_c + gt[:, 1:2] * o_s + gt[:, 2:3] * o_w)
                lse[b, i, g * G:(g + 1) * G, 0] = l_c
                lse[b, i, g * G:(g + 1) * G, 1] = l_s
                lse[b, i, g * G:(g + 1) * G, 2] = l_w
    return out, lse
