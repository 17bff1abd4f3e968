"""Pins for oracle.nsa (and the block log-sum-exp score of oracle.select) against
things other than themselves.

* round_bf16: hand-worked IEEE ties and an independent float32 -> bf16 rounding;
* compress: math.fsum means over scalar page lookups, and the nearest-bf16 property;
  complete blocks counted by enumeration; constant blocks compress exactly;
* nsa_attn: each branch alone (gates one-hot) against the scalar brute force over
  the positions the reading names (compressed rows, window + tail, blocks + tail),
  the gated sum by linearity, approximate grouping against a set-union brute force,
  empty branches (zero output, lse = -inf);
* block log-sum-exp: closed forms, scipy's logsumexp, and rank enumeration.
"""
import math

import numpy as np
import pytest

from long_context_self_amd import synth
from oracle import attention as oa
from oracle import brute
from oracle import nsa
from oracle import select as osel


def small(**kw):
    base = synth.Config("n", B=2, Hq=4, Hkv=2, d=16, L=96, page_size=8, n_q=4, n_draft=0, top_k=3,
                        n_sink=0, n_recent=0, mode="block", crit_frac=0.0, blocks_per_row=3, core_blocks=2,
                        tree_branches=2)
    return base.with_(**kw)


def test_round_bf16_hand_worked_ties():
    one = 1.0
    ulp = 2.0 ** -7                                   # bf16 spacing in [1, 2)
    cases = {one: 0x3F80, one + ulp / 2: 0x3F80,      # tie -> even (1.0)
             one + 3 * ulp / 2: 0x3F82,               # tie between 0x3F81 and 0x3F82 -> even
             one + ulp / 2 + 2.0 ** -30: 0x3F81,      # just above the tie
             -1.5: 0xBFC0, 0.0: 0x0000, 2.0 ** -20: 0x3580, 3.0: 0x4040}
    for x, bits in cases.items():
        assert int(nsa.round_bf16(np.array([x]))[0]) == bits, (x, hex(int(nsa.round_bf16(np.array([x]))[0])))


def test_round_bf16_agrees_with_float32_rounding_on_float32_inputs():
    """On values that are float32 already, rounding from float64 and from float32 agree
    (no double rounding); synth's integer-bias rounding is an independent routine."""
    rng = np.random.default_rng(1)
    x = (rng.standard_normal(20000) * np.exp(rng.uniform(-8, 8, 20000))).astype(np.float32)
    assert np.array_equal(nsa.round_bf16(x.astype(np.float64)), synth.f32_to_bf16_bits(x))


def test_n_compressed_by_enumeration():
    for L in range(0, 70):
        for l, s in ((8, 8), (8, 4), (16, 8), (32, 16), (4, 1)):
            assert nsa.n_compressed(L, l, s) == sum(1 for i in range(L + 1) if i * s + l <= L)


@pytest.mark.parametrize("l,s", [(8, 8), (16, 8), (8, 4)])
def test_compress_is_the_nearest_bf16_of_the_block_mean(l, s):
    cfg = small()
    kv = synth.make_paged_kv(cfg, seed=2, lens=[96, 41])
    kc, vc = nsa.compress(kv.k, kv.v, kv.block_table, kv.prefix_len, cfg.page_size, l, s)
    for b in range(cfg.B):
        n = nsa.n_compressed(int(kv.prefix_len[b]), l, s)
        assert np.all(kc[b, :, n:] == 0)
        for g in range(cfg.Hkv):
            for i in range(n):
                for cache, comp in ((kv.k, kc), (kv.v, vc)):
                    rows = [brute.row(cache, kv.block_table, b, g, p, cfg.page_size)
                            for p in range(i * s, i * s + l)]
                    for t in range(cfg.d):
                        mean = math.fsum(r[t] for r in rows) / l
                        bits = int(comp[b, g, i, t])
                        got = brute.bf16(bits)
                        # nearest bf16: neither neighbour (magnitude one step up or down;
                        # the smallest of either sign around zero) is closer to the mean
                        nbs = (0x0001, 0x8001) if bits & 0x7FFF == 0 else (bits - 1, bits + 1)
                        for nb in nbs:
                            assert abs(got - mean) <= abs(brute.bf16(nb) - mean)


def test_compress_constant_blocks_are_exact():
    cfg = small(B=1)
    kv = synth.make_paged_kv(cfg, seed=3)
    k = kv.k.copy()
    k[:] = 0x3FC0          # bf16 1.5 everywhere
    kc, _ = nsa.compress(k, kv.v, kv.block_table, kv.prefix_len, cfg.page_size, 16, 8)
    n = nsa.n_compressed(cfg.L, 16, 8)
    assert n == 11 and np.all(kc[0, :, :n] == 0x3FC0)


def _setup(seed=4, lens=(96, 57)):
    cfg = small()
    kv = synth.make_paged_kv(cfg, seed=seed, lens=list(lens), extra_tokens=cfg.n_q)
    q = synth.make_queries(cfg, kv, cfg.n_q, seed=seed)
    nblk = max(max(lens) // cfg.page_size, 12)
    sets = synth.make_block_sets(cfg, nblk, seed=seed)
    cnt = np.full(sets.shape[:3], sets.shape[3], dtype=np.int32)
    tm = np.stack([synth.tree_tail_masks(cfg.n_q, 2)] * cfg.B)
    return cfg, kv, q, sets, cnt, tm


def _gates(cfg, which):
    g = np.zeros((cfg.B, cfg.n_q, cfg.Hq, 3))
    g[..., which] = 1.0
    return g


def _vis_tail(tm, b, i, tb, tl):
    return [tb + j for j in range(tl) if (int(tm[b][i]) >> j) & 1]


def test_single_branches_match_brute_force():
    cfg, kv, q, sets, cnt, tm = _setup()
    l, s, window = 16, 8, 20
    scale = 1.0 / math.sqrt(cfg.d)
    kc, vc = nsa.compress(kv.k, kv.v, kv.block_table, kv.prefix_len, cfg.page_size, l, s)
    tl = np.full(cfg.B, cfg.n_q, dtype=np.int32)
    outs = {}
    for which in range(3):
        outs[which] = nsa.nsa_attn(q, kv.k, kv.v, kv.block_table, cfg.page_size, kc, vc, l, s, sets, cnt,
                                   kv.prefix_len, tl, window, _gates(cfg, which), scale, tail_mask=tm)
    for b in range(cfg.B):
        tb = int(kv.prefix_len[b])
        n = nsa.n_compressed(tb, l, s)
        # the compressed rows as a paged cache of one-token pages: page i = compressed row i
        ck = kc[b][:, :, None, :].transpose(1, 0, 2, 3)      # [M][Hkv][1][d]
        cv = vc[b][:, :, None, :].transpose(1, 0, 2, 3)
        cbt = np.arange(ck.shape[0], dtype=np.int32)[None, :]
        for i in range(cfg.n_q):
            tail = _vis_tail(tm, b, i, tb, cfg.n_q)
            for h in range(cfg.Hq):
                g = h // cfg.G
                o, lse_, _ = brute.attend(q[b, i, h], ck, cv, cbt, 0, g, list(range(n)), 1, scale)
                np.testing.assert_allclose(outs[0][0][b, i, h], o, rtol=0, atol=1e-12)
                assert abs(outs[0][1][b, i, h, 0] - lse_) < 1e-12
                blocks = sets[b, i, g, :cnt[b, i, g]]
                vis = [int(c) * cfg.page_size + t for c in blocks for t in range(cfg.page_size)
                       if int(c) * cfg.page_size + t < tb] + tail
                o, lse_, _ = brute.attend(q[b, i, h], kv.k, kv.v, kv.block_table, b, g, vis, cfg.page_size, scale)
                np.testing.assert_allclose(outs[1][0][b, i, h], o, rtol=0, atol=1e-12)
                assert abs(outs[1][1][b, i, h, 1] - lse_) < 1e-12
                vis = list(range(max(0, tb - window), tb)) + tail
                o, lse_, _ = brute.attend(q[b, i, h], kv.k, kv.v, kv.block_table, b, g, vis, cfg.page_size, scale)
                np.testing.assert_allclose(outs[2][0][b, i, h], o, rtol=0, atol=1e-12)
                assert abs(outs[2][1][b, i, h, 2] - lse_) < 1e-12


def test_gated_sum_is_linear_in_the_gates():
    cfg, kv, q, sets, cnt, tm = _setup(seed=5)
    l, s, window = 8, 8, 33
    scale = 1.0 / math.sqrt(cfg.d)
    kc, vc = nsa.compress(kv.k, kv.v, kv.block_table, kv.prefix_len, cfg.page_size, l, s)
    tl = np.full(cfg.B, cfg.n_q, dtype=np.int32)
    rng = np.random.default_rng(0)
    gates = rng.uniform(0, 1, (cfg.B, cfg.n_q, cfg.Hq, 3))
    out, lse = nsa.nsa_attn(q, kv.k, kv.v, kv.block_table, cfg.page_size, kc, vc, l, s, sets, cnt, kv.prefix_len,
                            tl, window, gates, scale, tail_mask=tm)
    parts = [nsa.nsa_attn(q, kv.k, kv.v, kv.block_table, cfg.page_size, kc, vc, l, s, sets, cnt, kv.prefix_len,
                          tl, window, _gates(cfg, c), scale, tail_mask=tm)[0] for c in range(3)]
    ref = sum(gates[..., c:c + 1] * parts[c] for c in range(3))
    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-12)
    # the selection branch with every row on its own blocks is block-mode sparse attention
    so, slse = oa.sparse_attn(q, kv.k, kv.v, kv.block_table, cfg.page_size, "block", sets, cnt, kv.prefix_len,
                              tl, scale, tail_mask=tm)
    np.testing.assert_allclose(parts[1], so, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse[..., 1], slse, rtol=0, atol=1e-12)


def test_approximate_grouping_uses_the_union_of_the_group():
    cfg, kv, q, sets, cnt, tm = _setup(seed=6)
    scale = 1.0 / math.sqrt(cfg.d)
    kc, vc = nsa.compress(kv.k, kv.v, kv.block_table, kv.prefix_len, cfg.page_size, 8, 8)
    tl = np.full(cfg.B, cfg.n_q, dtype=np.int32)
    out, _ = nsa.nsa_attn(q, kv.k, kv.v, kv.block_table, cfg.page_size, kc, vc, 8, 8, sets, cnt, kv.prefix_len,
                          tl, 0, _gates(cfg, 1), scale, tail_mask=tm, group="approximate")
    for b in range(cfg.B):
        tb = int(kv.prefix_len[b])
        for g in range(cfg.Hkv):
            union = set()
            for i in range(cfg.n_q):
                union |= {int(c) for c in sets[b, i, g, :cnt[b, i, g]]}
            assert len(union) > cfg.blocks_per_row            # the rows' sets really differ
            for i in range(cfg.n_q):
                vis = [c * cfg.page_size + t for c in sorted(union) for t in range(cfg.page_size)
                       if c * cfg.page_size + t < tb] + _vis_tail(tm, b, i, tb, cfg.n_q)
                for h in range(g * cfg.G, (g + 1) * cfg.G):
                    o, _, _ = brute.attend(q[b, i, h], kv.k, kv.v, kv.block_table, b, g, vis, cfg.page_size, scale)
                    np.testing.assert_allclose(out[b, i, h], o, rtol=0, atol=1e-12)


def test_empty_branches_contribute_nothing():
    cfg, kv, q, sets, cnt, tm = _setup(seed=7, lens=(12, 5))
    scale = 1.0 / math.sqrt(cfg.d)
    l, s = 16, 8                                   # prefixes shorter than one compressed block
    kc, vc = nsa.compress(kv.k, kv.v, kv.block_table, kv.prefix_len, cfg.page_size, l, s)
    tl = np.zeros(cfg.B, dtype=np.int32)           # no tail either
    cnt0 = np.zeros_like(cnt)
    out, lse = nsa.nsa_attn(q, kv.k, kv.v, kv.block_table, cfg.page_size, kc, vc, l, s, sets, cnt0,
                            kv.prefix_len, tl, 0, np.ones((cfg.B, cfg.n_q, cfg.Hq, 3)), scale, tail_mask=tm)
    assert np.all(out == 0) and np.all(np.isneginf(lse))


def test_block_lse_closed_forms_and_library():
    from scipy.special import logsumexp
    bs, L = 8, 29
    sig = np.full(L, 2.5)
    beta = osel.block_scores_lse(sig, L, bs)
    np.testing.assert_allclose(beta, [2.5 + math.log(8)] * 3 + [2.5 + math.log(5)], rtol=0, atol=1e-14)
    rng = np.random.default_rng(3)
    sig = rng.standard_normal(L) * 30
    beta = osel.block_scores_lse(sig, L, bs)
    ref = [logsumexp(sig[c * bs:min(L, c * bs + bs)]) for c in range(4)]
    np.testing.assert_allclose(beta, ref, rtol=1e-15, atol=1e-12)
    # a block dominated by one position scores that position's value (within log bs)
    assert np.all(beta >= osel.block_scores(sig, L, bs)) and np.all(beta <= osel.block_scores(sig, L, bs) + math.log(8))


@pytest.mark.parametrize("seed", range(3))
def test_block_lse_selection_matches_rank_enumeration(seed):
    rng = np.random.default_rng(300 + seed)
    bs, L = 8, int(rng.integers(60, 150))
    sig = rng.integers(-3, 4, size=L).astype(np.float64)
    k, ns, nr = 4, 3, 10
    got = osel.topk_blocks(sig, L, k, ns, nr, bs, agg="lse")
    nb = (L + bs - 1) // bs
    beta = [math.log(math.fsum(math.exp(x) for x in sig[c * bs:min(L, c * bs + bs)])) for c in range(nb)]
    sb, rb = (ns + bs - 1) // bs, (L - nr) // bs
    ref = list(range(sb)) + brute.topk_by_rank(beta, sb, rb, k) + list(range(rb, nb))
    assert got.tolist() == sorted(ref)


def test_block_lse_prefers_more_strong_positions_where_max_ties():
    # blocks of 4: block 1 holds one 5, block 2 four 5s; the max ties (smaller id wins),
    # the log-sum-exp counts the four
    sig = np.array([0, 0, 0, 0, 5, 0, 0, 0, 5, 5, 5, 5, 0, 0, 0, 0], dtype=np.float64)
    assert osel.topk_blocks(sig, 16, 1, 0, 0, 4).tolist() == [1]
    assert osel.topk_blocks(sig, 16, 1, 0, 0, 4, agg="lse").tolist() == [2]
