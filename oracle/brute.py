"""Pure-Python attention for tiny inputs (oracle pin; test infrastructure only).

Written independently of ``oracle.attention``: its own bf16 decode (through
``struct``), its own page lookup and scalar loops with ``math.fsum``.  It is
only meant for a few hundred positions.  It computes the plain definition of
softmax attention (Vegas page, "The pith": verification computes the exact
full-attention distribution).
"""
from __future__ import annotations

import math
import struct


def bf16(bits: int) -> float:
    return struct.unpack("<f", struct.pack("<I", (int(bits) & 0xFFFF) << 16))[0]


def row(cache, block_table, b: int, g: int, p: int, page_size: int):
    page = int(block_table[b][p // page_size])
    slot = p % page_size
    return [bf16(x) for x in cache[page][g][slot]]


def attend(q_bits, cache_k, cache_v, block_table, b: int, g: int, positions, page_size: int,
           scale: float):
    """One query row (bf16 bits [d]) over the given positions; returns (o, lse, logits)."""
    q = [bf16(x) for x in q_bits]
    logits = []
    vs = []
    for p in positions:
        k = row(cache_k, block_table, b, g, p, page_size)
        logits.append(scale * math.fsum(qi * ki for qi, ki in zip(q, k)))
        vs.append(row(cache_v, block_table, b, g, p, page_size))
    if not logits:
        return [0.0] * len(q), -math.inf, []
    m = max(logits)
    w = [math.exp(s - m) for s in logits]
    z = math.fsum(w)
    d = len(q)
    o = [math.fsum(w[t] * vs[t][c] for t in range(len(w))) / z for c in range(d)]
    return o, m + math.log(z), logits


def topk_by_rank(sigma, lo: int, hi: int, k: int):
    """Positions in [lo, hi) beaten by fewer than k others (greater score, or equal and smaller index)."""
    out = []
    for p in range(lo, hi):
        beaten = 0
        for r in range(lo, hi):
            if sigma[r] > sigma[p] or (sigma[r] == sigma[p] and r < p):
                beaten += 1
        if beaten < k:
            out.append(p)
    return out
