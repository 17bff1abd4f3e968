"""Pins for oracle.select against things other than itself.

* pairwise rank enumeration (oracle.brute.topk_by_rank) on small inputs with
  many ties: a position is kept iff fewer than k pool positions beat it;
* invariants: budget size, sink and recent windows present, every chosen score
  >= every unchosen pool score, ascending output;
* the pinned float32 order, checked on inputs whose IEEE results are worked
  out by hand (absorption at 2**24) and on dyadic inputs where float32 is exact;
* the float32 score stays within the standard error bound of the float64 one.
"""
import math

import numpy as np
import pytest

from long_context_self_amd import synth
from oracle import attention as oa
from oracle import brute
from oracle import select as osel


@pytest.mark.parametrize("seed", range(6))
def test_topk_tokens_matches_rank_enumeration(seed):
    rng = np.random.default_rng(seed)
    L = int(rng.integers(20, 64))
    sig = rng.integers(-4, 5, size=L).astype(np.float64)   # many ties
    k, ns, nr = 7, 2, 3
    got = osel.topk_tokens(sig, L, k, ns, nr)
    ref = list(range(ns)) + brute.topk_by_rank(sig, ns, L - nr, k) + list(range(L - nr, L))
    assert got.tolist() == sorted(ref)


def test_topk_tokens_invariants():
    rng = np.random.default_rng(11)
    for _ in range(50):
        L = int(rng.integers(1, 300))
        k, ns, nr = int(rng.integers(0, 40)), int(rng.integers(0, 6)), int(rng.integers(0, 20))
        sig = rng.standard_normal(L)
        out = osel.topk_tokens(sig, L, k, ns, nr)
        assert np.all(np.diff(out) > 0)
        if L <= ns + k + nr:
            assert out.tolist() == list(range(L))
            continue
        assert out.size == ns + k + nr
        s = set(out.tolist())
        assert all(p in s for p in range(ns)) and all(p in s for p in range(L - nr, L))
        pool = np.arange(ns, L - nr)
        chosen = np.array([p for p in pool if p in s])
        unchosen = np.array([p for p in pool if p not in s])
        if chosen.size and unchosen.size:
            assert sig[chosen].min() >= sig[unchosen].max()


@pytest.mark.parametrize("seed", range(4))
def test_topk_blocks_matches_rank_enumeration(seed):
    rng = np.random.default_rng(100 + seed)
    bs = 8
    L = int(rng.integers(40, 200))
    sig = rng.integers(-3, 4, size=L).astype(np.float32)
    k, ns, nr = 4, 3, 10
    got = osel.topk_blocks(sig, L, k, ns, nr, bs)
    nb = (L + bs - 1) // bs
    beta = [max(sig[c * bs:min(L, c * bs + bs)]) for c in range(nb)]
    sb = (ns + bs - 1) // bs                  # blocks holding a sink position
    rb = (L - nr) // bs                       # first block that meets the recent window
    ref = list(range(sb)) + brute.topk_by_rank(beta, sb, rb, k) + list(range(rb, nb))
    assert got.tolist() == sorted(ref)
    # every always-kept block really holds a sink or recent position
    for c in list(range(sb)) + list(range(rb, nb)):
        lo, hi = c * bs, min(L, c * bs + bs)
        assert lo < ns or hi > L - nr


def test_blocks_short_context_keeps_all():
    sig = np.arange(30, dtype=np.float32)
    assert osel.topk_blocks(sig, 30, 2, 4, 4, 8).tolist() == [0, 1, 2, 3]


def test_pinned_order_absorption():
    """Worked IEEE example: 2**24 + 1 rounds back to 2**24 (ties to even) in float32.

    Heads in ascending order contribute pairs (2**24, 0), (1, 0), (1, 0):
    pinned float32 order gives 2**24 after each step; float64 gives 2**24 + 2.
    Reversed order would give 2 + 2**24 = 2**24 + 2 (exact in float32).
    """
    lg = np.zeros((1, 3, 2, 1), dtype=np.float32)
    lg[0, 0, 0, 0] = 2.0 ** 24
    lg[0, 1, 0, 0] = 1.0
    lg[0, 2, 0, 0] = 1.0
    s32 = osel.scores_f32_pinned(lg, 0, 1, [0, 1, 2])
    assert s32[0] == np.float32(2.0 ** 24)
    assert osel.scores_f64(lg, 0, 1, [0, 1, 2])[0] == 2.0 ** 24 + 2


def test_pinned_pair_first():
    """Each (row0, row1) pair is rounded before it joins the accumulator.

    pair (2**24, 1) -> 2**24; then + (1, 1) = 2 -> 2**24 + 2 exactly.
    Summing row by row across heads instead would differ.
    """
    lg = np.zeros((1, 2, 2, 1), dtype=np.float32)
    lg[0, 0, 0, 0], lg[0, 0, 1, 0] = 2.0 ** 24, 1.0
    lg[0, 1, 0, 0], lg[0, 1, 1, 0] = 1.0, 1.0
    assert osel.scores_f32_pinned(lg, 0, 1, [0, 1])[0] == np.float32(2.0 ** 24 + 2)


def test_negative_zero_canonical():
    lg = np.zeros((1, 1, 2, 3), dtype=np.float32)
    lg[0, 0, 0, 1] = -0.0
    lg[0, 0, 1, 1] = -0.0
    s = osel.scores_f32_pinned(lg, 0, 3, [0])
    assert not np.signbit(s).any()


def test_f32_exact_on_dyadic_and_within_bound():
    rng = np.random.default_rng(5)
    # dyadic values with few bits: every partial sum is exact in float32
    lg = (rng.integers(-64, 64, size=(2, 8, 2, 50)) / 8.0).astype(np.float32)
    for b in range(2):
        np.testing.assert_array_equal(osel.scores_f32_pinned(lg, b, 50, range(8)).astype(np.float64),
                                      osel.scores_f64(lg, b, 50, range(8)))
    # generic values: |f32 - f64| <= n * eps32 * sum|terms| (recursive summation bound)
    lg = rng.standard_normal((1, 32, 2, 400)).astype(np.float32) * 5
    s32 = osel.scores_f32_pinned(lg, 0, 400, range(32)).astype(np.float64)
    s64 = osel.scores_f64(lg, 0, 400, range(32))
    bound = 64 * np.finfo(np.float32).eps * np.abs(lg[0].astype(np.float64)).sum(axis=(0, 1))
    assert np.all(np.abs(s32 - s64) <= bound)


def test_set_heads_group_membership():
    """Per-KV-head sets see only their own group's heads: a spike planted in one
    group's logits is selected for that group only."""
    B, Hq, Hkv, L = 1, 8, 4, 100
    lg = np.zeros((B, Hq, 2, L), dtype=np.float32)
    rng = np.random.default_rng(0)
    lg[:] = rng.standard_normal(lg.shape) * 0.01
    lg[0, 4:6, :, 50] = 10.0       # heads 4,5 = group 2
    res = osel.select(lg, np.array([L]), Hkv, "per_kv_head", top_k=1, n_sink=0, n_recent=0)
    assert res[0][2].tolist() == [50]
    for g in (0, 1, 3):
        assert 50 not in res[0][g].tolist()
    shared = osel.select(lg, np.array([L]), Hkv, "shared", top_k=1, n_sink=0, n_recent=0)
    assert shared[0][0].tolist() == [50]


def test_planted_critical_recall_tiny():
    """Quality sanity, not parity: on the tiny workload the selector recovers most
    planted critical keys from the two verifier rows."""
    cfg = synth.CONFIGS["tiny"]
    kv = synth.make_paged_kv(cfg, seed=0)
    q = synth.make_queries(cfg, kv, cfg.n_q, seed=0)
    _, logits, _ = oa.verify_attn(q, kv.k, kv.v, kv.block_table, kv.prefix_len, cfg.page_size,
                                  1.0 / math.sqrt(cfg.d))
    sel = osel.select(logits, kv.prefix_len, cfg.Hkv, "shared", cfg.top_k, cfg.n_sink, cfg.n_recent)
    chosen = set(sel[0][0].tolist())
    assert len(chosen) == cfg.top_k + cfg.n_sink + cfg.n_recent
    crit = set(np.concatenate(kv.critical[0]).tolist())
    recall = len(crit & chosen) / len(crit)
    assert recall > 0.6


@pytest.mark.parametrize("n_rows", [1, 3, 9])
def test_pinned_n_rows_exact_on_small_integers(n_rows):
    """Small integers add exactly in float32 in any order, so the pinned n-row score
    must equal the exact integer sum over heads and rows (a dropped row, head or
    term, or a wrong axis, changes it)."""
    rng = np.random.default_rng(n_rows)
    B, Hq, L = 2, 6, 50
    lg = rng.integers(-1000, 1000, size=(B, Hq, n_rows, L)).astype(np.float32)
    for b in range(B):
        for heads in ([0, 1, 2, 3, 4, 5], [2, 3]):
            exact = lg[b, heads].astype(np.int64).sum(axis=(0, 1))
            got = osel.scores_f32_pinned(lg, b, L, heads)
            assert np.array_equal(got.astype(np.int64), exact)


def test_pinned_n_rows_order():
    """Within a head the rows are summed first, left to right: (((a + b) + c)) with
    a = 2^24, b = c = 1 gives 2^24 (each 1 is absorbed), not 2^24 + 2."""
    lg = np.zeros((1, 1, 3, 1), dtype=np.float32)
    lg[0, 0, :, 0] = [2.0 ** 24, 1.0, 1.0]
    assert osel.scores_f32_pinned(lg, 0, 1, [0])[0] == np.float32(2.0 ** 24)
    lg[0, 0, :, 0] = [1.0, 1.0, 2.0 ** 24]
    assert osel.scores_f32_pinned(lg, 0, 1, [0])[0] == np.float32(2.0 ** 24 + 2)


def test_weights_closed_form_uniform_keys():
    """Every key equal: row r of a chain sees L + r + 1 positions with equal weight, so
    each prefix position scores sum over heads and collected rows of 1/(L + r + 1)."""
    cfg = synth.Config("w", B=2, Hq=4, Hkv=2, d=16, L=40, page_size=8, n_q=4, n_draft=3,
                       top_k=8, n_sink=2, n_recent=3, mode="shared", crit_frac=0.0)
    kv = synth.make_paged_kv(cfg, seed=5, lens=[40, 23])
    kv.k[...] = kv.k[0, 0, 0, :]                        # one key row everywhere
    q = synth.make_queries(cfg, kv, cfg.n_q, seed=5)
    rows = [3, 0, 2]
    _, logits, lse = oa.verify_attn(q, kv.k, kv.v, kv.block_table, kv.prefix_len, cfg.page_size, 0.25,
                                    collect_rows=rows)
    for b in range(cfg.B):
        L = int(kv.prefix_len[b])
        for heads in (list(range(cfg.Hq)), [2, 3]):
            got = osel.scores_weights_f64(logits, lse, rows, b, L, heads)
            want = len(heads) * sum(1.0 / (L + r + 1) for r in rows)
            np.testing.assert_allclose(got, want, rtol=1e-12, atol=0)


def test_weights_mass_matches_softmax_weights():
    """Per head, the weight scores over the prefix sum to the rows' prefix mass, which
    the attention oracle's normalised weights give independently (one minus the mass
    on the verifier tail)."""
    cfg = synth.Config("w", B=1, Hq=4, Hkv=2, d=16, L=33, page_size=4, n_q=5, n_draft=4,
                       top_k=8, n_sink=2, n_recent=3, mode="shared", crit_frac=0.05)
    kv = synth.make_paged_kv(cfg, seed=6)
    q = synth.make_queries(cfg, kv, cfg.n_q, seed=6)
    rows = [0, 4, 2]
    _, logits, lse, W = oa.verify_attn(q, kv.k, kv.v, kv.block_table, kv.prefix_len, cfg.page_size, 0.25,
                                       collect_rows=rows, return_weights=True)
    L = int(kv.prefix_len[0])
    for h in range(cfg.Hq):
        g, hh = divmod(h, cfg.G)
        got = osel.scores_weights_f64(logits, lse, rows, 0, L, [h]).sum()
        want = sum(W[(0, g)][r, hh, :L].sum() for r in rows)
        assert abs(got - want) < 1e-12
        assert got < len(rows)


def test_partial_scores_group_first_association():
    """Shared selection from per-KV-head partials sums each group first: heads
    (2^24, 1 | 1, 1) give 2^24 + 2 grouped but 2^24 flat (every 1 absorbed in turn)."""
    lg = np.zeros((1, 4, 2, 1), dtype=np.float32)
    lg[0, :, 0, 0] = [2.0 ** 24, 1.0, 1.0, 1.0]
    part = osel.partial_scores_f32(lg, 0, 1, 4, 2)
    assert part[:, 0].tolist() == [2.0 ** 24, 2.0]
    grouped = osel.scores_f32_pinned(part[None, :, None, :], 0, 1, [0, 1])
    flat = osel.scores_f32_pinned(lg, 0, 1, [0, 1, 2, 3])
    assert grouped[0] == np.float32(2.0 ** 24 + 2) and flat[0] == np.float32(2.0 ** 24)


def test_partial_scores_exact_on_small_integers():
    rng = np.random.default_rng(11)
    B, Hq, Hkv, L = 2, 12, 3, 40
    lg = rng.integers(-500, 500, size=(B, Hq, 2, L)).astype(np.float32)
    for b in range(B):
        part = osel.partial_scores_f32(lg, b, L, Hq, Hkv)
        want = lg[b].astype(np.int64).reshape(Hkv, Hq // Hkv, 2, L).sum(axis=(1, 2))
        assert np.array_equal(part.astype(np.int64), want)


@pytest.mark.parametrize("seed", range(3))
def test_select_block_mode_per_group_matches_rank_enumeration(seed):
    """select(mode='block') end to end: one block set per (sequence, KV head), each scored
    by the max over its block of the group's own head sum (math.fsum over the G heads'
    two rows), kept by rank enumeration between the sink and recent windows.  Summing the
    wrong heads (all heads, or group 0's for every set) fails here."""
    rng = np.random.default_rng(200 + seed)
    B, Hq, Hkv, bs = 2, 6, 3, 8
    G = Hq // Hkv
    lens = [int(rng.integers(60, 120)), int(rng.integers(60, 120))]
    ld = max(lens)
    # small integers: many ties between blocks, and group sums that differ per group
    lg = rng.integers(-3, 4, size=(B, Hq, 2, ld)).astype(np.float64)
    k, ns, nr = 3, 5, 11
    got = osel.select(lg, np.array(lens), Hkv, "block", k, ns, nr, block_size=bs)
    for b in range(B):
        L = lens[b]
        nb = (L + bs - 1) // bs
        sb = (ns + bs - 1) // bs
        rb = (L - nr) // bs
        for g in range(Hkv):
            sig = [math.fsum(lg[b, h, c, p] for h in range(g * G, (g + 1) * G) for c in range(2))
                   for p in range(L)]
            beta = [max(sig[c * bs:min(L, c * bs + bs)]) for c in range(nb)]
            ref = list(range(sb)) + brute.topk_by_rank(beta, sb, rb, k) + list(range(rb, nb))
            assert got[b][g].tolist() == sorted(ref), (b, g)
    # the groups really select differently on these inputs (so the test can tell them apart)
    assert any(got[b][0].tolist() != got[b][g].tolist() for b in range(B) for g in range(1, Hkv))


def test_to_physical_hand_worked_and_round_trip():
    bt = np.array([[3, 0, 2, 1]], dtype=np.int32)     # logical page i lives in physical page bt[0][i]
    P = 4
    assert osel.to_physical(np.array([0, 5, 9, 15]), bt, 0, P).tolist() == [12, 1, 9, 7]
    rng = np.random.default_rng(9)
    bt = rng.permutation(64).astype(np.int32)[None, :]
    pos = np.sort(rng.choice(64 * 16, 100, replace=False))
    phys = osel.to_physical(pos, bt, 0, 16)
    inv = np.argsort(bt[0])                              # physical page -> logical page
    assert np.array_equal(inv[phys // 16] * 16 + phys % 16, pos)
