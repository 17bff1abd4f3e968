"""Seeded synthetic workloads for the verify / select / sparse-draft attention path.

This module only draws inputs.  It holds none of the method's arithmetic: no
attention, no scoring, no top-k.  Both the CPU oracle (through the tests) and
the GPU path consume exactly the arrays produced here, so it is the one piece
of code the two sides share.

Workload recipe (the pages fix the shapes, not the data; the data are ours):

* Q, K, V entries are N(0, 1) drawn in float32 and rounded to bfloat16 with
  round-to-nearest-even.
* For every (sequence b, KV head g) a unit direction ``u = z / |z|`` with
  ``z ~ N(0, I_d)`` is drawn.  A critical set of ``floor(f * L)`` prefix
  positions is drawn uniformly without replacement; their keys get ``+3 u``
  before rounding.  Every query of a head in group g gets ``+sqrt(d) u``.  A
  critical key therefore scores about +3 above the background logit, whose
  standard deviation is about sqrt(2).  This stands in for the "few critical
  KV entries" whose existence the Vegas and Sparse Glimpse pages rely on.
* The KV cache is paged: K and V are bf16 arrays ``[num_pages][Hkv][P][d]``,
  and ``block_table[b][i]`` names the physical page of logical page i of
  sequence b.  Pages are a seeded random permutation, so paging is exercised.
* Each sequence's cache holds its prefix (``prefix_len[b]`` tokens), then the
  ``n_q`` verifier tokens, then ``n_draft`` draft tokens.  Slots past that in
  the last page are filled with NaN so that a kernel which reads an unused
  slot into a result is caught.

Shapes follow the workloads quoted on the pages (long-context inputs of
96K-120K tokens for Vegas, up to 64K for Sparse Glimpse, 8K/32K for SSV); no
dataset item is used or reproduced.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, List, Optional, Sequence

import numpy as np

BF16_NAN = np.uint16(0x7FC0)


# ----------------------------------------------------------------------------
# bf16 bit handling (input preparation only)
# ----------------------------------------------------------------------------

def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (round to nearest, ties to even); return uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    r = ((u + bias) >> np.uint32(16)).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        r[nan] = BF16_NAN
    return r


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bits to float32."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


# ----------------------------------------------------------------------------
# configurations
# ----------------------------------------------------------------------------

@dataclasses.dataclass(frozen=True)
class Config:
    name: str
    B: int
    Hq: int
    Hkv: int
    d: int
    L: int                 # prefix length per sequence
    page_size: int
    n_q: int               # verifier rows = draft length + 1 (bonus token)
    n_draft: int           # single-token draft steps per iteration
    top_k: int
    n_sink: int
    n_recent: int
    mode: str              # 'shared' | 'per_kv_head' | 'block'
    crit_frac: float
    # block-sparse (SSV) extras: per-row block sets drawn with a shared core
    blocks_per_row: int = 0
    core_blocks: int = 0
    tree_branches: int = 0  # >0: n_q rows form this many root chains
    # NSA branches (SSV sparse verification): compression block length and stride,
    # sliding-window length.  The pages name the branches without sizes; these are
    # NSA's published sizes (blocks of 32 at stride 16, a 512-token window).
    cmp_len: int = 0
    cmp_stride: int = 0
    window: int = 0

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv

    @property
    def collect_rows(self):
        return (0, self.n_q - 1)

    def with_(self, **kw) -> "Config":
        return dataclasses.replace(self, **kw)


CONFIGS: Dict[str, Config] = {
    # Tiny: B1, 4/2 heads, d64, L1024, 1% critical, draft 4 (5 verifier rows),
    # top-k 64 + 4 sink + 16 recent.
    "tiny": Config("tiny", B=1, Hq=4, Hkv=2, d=64, L=1024, page_size=16, n_q=5,
                   n_draft=4, top_k=64, n_sink=4, n_recent=16, mode="shared",
                   crit_frac=0.01),
    # Llama-3-8B-shaped layer at 32K context, draft 8 (rows 0 and 8 collected).
    "llama8b_32k": Config("llama8b_32k", B=1, Hq=32, Hkv=8, d=128, L=32768,
                          page_size=16, n_q=9, n_draft=8, top_k=2048, n_sink=4,
                          n_recent=64, mode="shared", crit_frac=0.005),
    # 14B-shaped layer, B4 at 64K, per-KV-head index (Sparse Glimpse variant).
    "qwen14b_64k": Config("qwen14b_64k", B=4, Hq=40, Hkv=8, d=128, L=65536,
                          page_size=16, n_q=7, n_draft=6, top_k=4096, n_sink=4,
                          n_recent=128, mode="per_kv_head", crit_frac=0.0025),
    # NSA-style blockwise (SSV): 64-token blocks, 16 per verifier row, a
    # depth-4 x branching-2 draft tree (8 rows), ~60% pairwise block overlap.
    "nsa_16k": Config("nsa_16k", B=2, Hq=32, Hkv=8, d=128, L=16384,
                      page_size=64, n_q=8, n_draft=0, top_k=16, n_sink=0,
                      n_recent=0, mode="block", crit_frac=0.0,
                      blocks_per_row=16, core_blocks=10, tree_branches=2,
                      cmp_len=32, cmp_stride=16, window=512),
    # Long-context stress: B8 at 128K, draft 8, 4096 + 4 + 64.
    "stress_128k": Config("stress_128k", B=8, Hq=32, Hkv=8, d=128, L=131072,
                          page_size=16, n_q=9, n_draft=8, top_k=4096, n_sink=4,
                          n_recent=64, mode="shared", crit_frac=0.001),
}


# ----------------------------------------------------------------------------
# generators
# ----------------------------------------------------------------------------

def _rng(seed: int, *tag: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([int(seed), *[int(t) for t in tag]]))


@dataclasses.dataclass
class PagedKV:
    k: np.ndarray            # uint16 bf16 bits [num_pages][Hkv][P][d]
    v: np.ndarray            # uint16 bf16 bits [num_pages][Hkv][P][d]
    block_table: np.ndarray  # int32 [B][max_pages]
    prefix_len: np.ndarray   # int32 [B]
    cache_len: np.ndarray    # int32 [B] tokens actually written per sequence
    u: np.ndarray            # float32 [B][Hkv][d] planted directions
    critical: List[List[np.ndarray]]  # [b][g] -> sorted int64 positions
    page_size: int

    @property
    def num_pages(self) -> int:
        return self.k.shape[0]

    @property
    def max_pages(self) -> int:
        return self.block_table.shape[1]


def make_paged_kv(cfg: Config, seed: int = 0, lens: Optional[Sequence[int]] = None,
                  extra_tokens: Optional[int] = None, poison_tail: bool = True) -> PagedKV:
    """Draw a paged bf16 KV cache holding, per sequence, prefix + verifier + draft tokens."""
    B, Hkv, d, P = cfg.B, cfg.Hkv, cfg.d, cfg.page_size
    lens = np.asarray(lens if lens is not None else [cfg.L] * B, dtype=np.int64)
    assert lens.shape == (B,)
    extra = cfg.n_q + cfg.n_draft if extra_tokens is None else extra_tokens
    cache_len = lens + extra
    pages_per_seq = [(int(n) + P - 1) // P for n in cache_len]
    max_pages = max(1, max(pages_per_seq))
    num_pages = max(1, sum(pages_per_seq))

    rng_u = _rng(seed, 1)
    z = rng_u.standard_normal((B, Hkv, d), dtype=np.float32)
    u = (z / np.linalg.norm(z, axis=-1, keepdims=True)).astype(np.float32)

    perm = _rng(seed, 2).permutation(num_pages).astype(np.int32)
    block_table = np.full((B, max_pages), -1, dtype=np.int32)
    # unused block-table slots point at page 0 but are never addressed
    block_table[:] = 0
    off = 0
    for b in range(B):
        n = pages_per_seq[b]
        block_table[b, :n] = perm[off:off + n]
        off += n

    k = np.empty((num_pages, Hkv, P, d), dtype=np.uint16)
    v = np.empty((num_pages, Hkv, P, d), dtype=np.uint16)
    critical: List[List[np.ndarray]] = []
    for b in range(B):
        n_tok = int(cache_len[b])
        n_pg = pages_per_seq[b]
        rng_kv = _rng(seed, 3, b)
        crit_b = []
        # logical [n_pg*P][Hkv][d] in float32, drawn page by page to bound memory
        chunk_pages = max(1, (1 << 22) // max(1, Hkv * P * d))
        n_crit = int(math.floor(cfg.crit_frac * int(lens[b])))
        crit_sets = []
        for g in range(Hkv):
            rc = _rng(seed, 4, b, g)
            cs = np.sort(rc.choice(int(lens[b]), size=n_crit, replace=False)) if n_crit > 0 \
                else np.zeros(0, dtype=np.int64)
            crit_sets.append(cs.astype(np.int64))
        crit_b = crit_sets
        for p0 in range(0, n_pg, chunk_pages):
            p1 = min(n_pg, p0 + chunk_pages)
            kk = rng_kv.standard_normal(((p1 - p0), Hkv, P, d), dtype=np.float32)
            vv = rng_kv.standard_normal(((p1 - p0), Hkv, P, d), dtype=np.float32)
            t0, t1 = p0 * P, p1 * P
            for g in range(Hkv):
                cs = crit_sets[g]
                sel = cs[(cs >= t0) & (cs < t1)] - t0
                if sel.size:
                    pg, sl = sel // P, sel % P
                    kk[pg, g, sl, :] += 3.0 * u[b, g]
            kb = f32_to_bf16_bits(kk)
            vb = f32_to_bf16_bits(vv)
            if poison_tail and t1 > n_tok:
                # slots past the written tokens of the last page
                lo = n_tok - t0
                flat_k = kb.reshape(p1 - p0, Hkv, P, d)
                for t in range(lo, t1 - t0):
                    flat_k[t // P, :, t % P, :] = BF16_NAN
                    vb[t // P, :, t % P, :] = BF16_NAN
            phys = block_table[b, p0:p1]
            k[phys] = kb
            v[phys] = vb
        critical.append(crit_b)
    return PagedKV(k=k, v=v, block_table=block_table, prefix_len=lens.astype(np.int32),
                   cache_len=cache_len.astype(np.int32), u=u, critical=critical, page_size=P)


def make_queries(cfg: Config, kv: PagedKV, n_rows: int, seed: int = 0, tag: int = 0) -> np.ndarray:
    """bf16 bits [B][n_rows][Hq][d]: N(0,1) plus sqrt(d) times the group's planted direction."""
    B, Hq, d, G = cfg.B, cfg.Hq, cfg.d, cfg.G
    rng = _rng(seed, 5, tag)
    q = rng.standard_normal((B, n_rows, Hq, d), dtype=np.float32)
    shift = np.repeat(kv.u, G, axis=1) * np.float32(math.sqrt(d))  # [B][Hq][d]
    q += shift[:, None, :, :]
    return f32_to_bf16_bits(q)


def chain_tail_masks(n_q: int) -> np.ndarray:
    """Row i sees verifier tokens 0..i (a plain draft chain)."""
    return np.array([(1 << (i + 1)) - 1 for i in range(n_q)], dtype=np.uint64)


def tree_tail_masks(n_q: int, branches: int) -> np.ndarray:
    """``branches`` chains of equal depth hanging off the last prefix token.

    Node j of chain c sits at verifier slot c*depth + j and sees its ancestors
    in the same chain and itself.
    """
    assert n_q % branches == 0
    depth = n_q // branches
    m = np.zeros(n_q, dtype=np.uint64)
    for c in range(branches):
        for j in range(depth):
            bits = 0
            for a in range(j + 1):
                bits |= 1 << (c * depth + a)
            m[c * depth + j] = bits
    return m


def make_block_sets(cfg: Config, n_blocks: int, seed: int = 0) -> np.ndarray:
    """Per (b, row, KV head) sorted block ids: a shared core plus private blocks.

    ``core_blocks`` ids are shared by all rows of a (b, g) pair and each row adds
    ``blocks_per_row - core_blocks`` private ids, all distinct, drawn without
    replacement from ``n_blocks``.  Pairwise overlap is core/blocks_per_row.
    Returns int32 [B][n_q][Hkv][blocks_per_row].
    """
    B, n_q, Hkv = cfg.B, cfg.n_q, cfg.Hkv
    kb, core = cfg.blocks_per_row, cfg.core_blocks
    priv = kb - core
    need = core + n_q * priv
    assert need <= n_blocks, "not enough blocks for distinct private sets"
    out = np.empty((B, n_q, Hkv, kb), dtype=np.int32)
    for b in range(B):
        for g in range(Hkv):
            r = _rng(seed, 6, b, g)
            ids = r.choice(n_blocks, size=need, replace=False)
            c = ids[:core]
            for i in range(n_q):
                p = ids[core + i * priv: core + (i + 1) * priv]
                out[b, i, g] = np.sort(np.concatenate([c, p]))
    return out


def make_gates(cfg: Config, n_rows: int, seed: int = 0) -> np.ndarray:
    """float32 [B][n_rows][Hq][3] branch gates, uniform in [0, 1) (NSA's gates are sigmoids)."""
    return _rng(seed, 9).uniform(0.0, 1.0, (cfg.B, n_rows, cfg.Hq, 3)).astype(np.float32)


def make_compressed_cache(cfg: Config, max_cmp: int, seed: int = 0):
    """bf16 bits [B][Hkv][max_cmp][d] x 2: stand-in compressed keys and values, N(0, 1)."""
    r = _rng(seed, 10)
    shape = (cfg.B, cfg.Hkv, max_cmp, cfg.d)
    return (f32_to_bf16_bits(r.standard_normal(shape, dtype=np.float32)),
            f32_to_bf16_bits(r.standard_normal(shape, dtype=np.float32)))


def drift_critical(cfg: Config, kv: PagedKV, frac: float, seed: int, it: int) -> List[List[np.ndarray]]:
    """Move ``frac`` of each (b, g) critical set to fresh prefix positions.

    Returns the new critical sets; :func:`rewrite_keys` then redraws the K rows
    of the positions that changed.  Models critical entries that change between
    speculative iterations of the long-context loop.
    """
    new = []
    for b in range(cfg.B):
        L = int(kv.prefix_len[b])
        row = []
        for g in range(cfg.Hkv):
            cs = kv.critical[b][g]
            r = _rng(seed, 7, it, b, g)
            n_move = int(round(frac * cs.size))
            if n_move == 0 or cs.size >= L:
                row.append(cs)
                continue
            keep = np.sort(r.choice(cs.size, size=cs.size - n_move, replace=False))
            taken = set(cs.tolist())
            fresh = []
            while len(fresh) < n_move:          # rejection: the set is a small fraction of L
                for p in r.integers(0, L, size=2 * n_move):
                    if len(fresh) < n_move and int(p) not in taken:
                        taken.add(int(p))
                        fresh.append(int(p))
            row.append(np.sort(np.concatenate([cs[keep], np.asarray(fresh, dtype=np.int64)])))
        new.append(row)
    return new


def rewrite_keys(cfg: Config, kv: PagedKV, new_sets: List[List[np.ndarray]], seed: int, it: int):
    """Redraw the K rows of positions that left or joined a critical set.

    A position that leaves gets a fresh N(0, 1) key; one that joins gets a fresh
    N(0, 1) key plus ``3 u``.  ``kv.k`` and ``kv.critical`` are updated in place.
    Returns (rows, bits): flat row ids into ``k.reshape(-1, d)`` and the new bf16
    rows, so that a device copy of the cache can be updated with one scatter.
    """
    P, d, Hkv = cfg.page_size, cfg.d, cfg.Hkv
    rows, bits = [], []
    for b in range(cfg.B):
        for g in range(Hkv):
            old, new = kv.critical[b][g], new_sets[b][g]
            changed = np.setxor1d(old, new)
            if changed.size == 0:
                continue
            x = _rng(seed, 8, it, b, g).standard_normal((changed.size, d), dtype=np.float32)
            join = np.isin(changed, new)
            x[join] += np.float32(3.0) * kv.u[b, g]
            kb = f32_to_bf16_bits(x)
            phys = kv.block_table[b, changed // P].astype(np.int64)
            slot = changed % P
            kv.k[phys, g, slot, :] = kb
            rows.append((phys * Hkv + g) * P + slot)
            bits.append(kb)
            kv.critical[b][g] = new
    if not rows:
        return np.zeros(0, dtype=np.int64), np.zeros((0, d), dtype=np.uint16)
    return np.concatenate(rows), np.concatenate(bits)
