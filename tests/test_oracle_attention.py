"""Pins for oracle.attention against things other than itself.

* brute force: pure-Python scalar loops with math.fsum (oracle.brute);
* a library routine: torch's CPU float64 scaled_dot_product_attention with an
  explicit boolean mask;
* closed forms: K = 0 gives the mean of the visible V rows, V = 1 gives 1, a
  single dominant key returns its V row;
* invariants: softmax rows sum to 1; sparse attention with every position
  selected equals dense attention.
"""
import math

import numpy as np
import pytest

from long_context_self_amd import synth
from oracle import attention as oa
from oracle import brute


def small_cfg(**kw):
    base = synth.Config("t", B=2, Hq=4, Hkv=2, d=16, L=37, page_size=4, n_q=3, n_draft=2,
                        top_k=8, n_sink=2, n_recent=3, mode="shared", crit_frac=0.05)
    return base.with_(**kw)


def make(cfg, seed=0, lens=None):
    kv = synth.make_paged_kv(cfg, seed=seed, lens=lens)
    q = synth.make_queries(cfg, kv, cfg.n_q, seed=seed)
    return kv, q


@pytest.mark.parametrize("tree", [False, True])
def test_verify_matches_brute_force(tree):
    cfg = small_cfg(n_q=4)
    kv, q = make(cfg, seed=3, lens=[37, 21])
    scale = 1.0 / math.sqrt(cfg.d)
    tm = None
    if tree:
        tm = np.stack([synth.tree_tail_masks(4, 2)] * cfg.B)
    out, logits, lse = oa.verify_attn(q, kv.k, kv.v, kv.block_table, kv.prefix_len,
                                      cfg.page_size, scale, tree_mask=tm)
    G = cfg.G
    for b in range(cfg.B):
        L = int(kv.prefix_len[b])
        for i in range(cfg.n_q):
            for h in range(cfg.Hq):
                if tm is None:
                    vis = list(range(L + i + 1))
                else:
                    vis = list(range(L)) + [L + j for j in range(cfg.n_q) if (int(tm[b][i]) >> j) & 1]
                o, l, lg = brute.attend(q[b, i, h], kv.k, kv.v, kv.block_table, b, h // G, vis,
                                        cfg.page_size, scale)
                np.testing.assert_allclose(out[b, i, h], o, rtol=0, atol=1e-12)
                assert abs(lse[b, i, h] - l) < 1e-12
                if i in (0, cfg.n_q - 1):
                    c = 0 if i == 0 else 1
                    np.testing.assert_allclose(logits[b, h, c, :L], lg[:L], rtol=0, atol=1e-12)
        # columns past the prefix are not written
        assert np.all(np.isnan(logits[b, :, :, int(kv.prefix_len[b]):]))


def test_verify_matches_torch_sdpa():
    torch = pytest.importorskip("torch")
    cfg = small_cfg(B=1, Hq=8, Hkv=2, d=32, L=50, page_size=8, n_q=5)
    kv, q = make(cfg, seed=1)
    scale = 1.0 / math.sqrt(cfg.d)
    out, logits, lse = oa.verify_attn(q, kv.k, kv.v, kv.block_table, kv.prefix_len,
                                      cfg.page_size, scale)
    L = cfg.L
    n = L + cfg.n_q
    # dense logical K/V [Hkv][n][d] from the paged cache, built by direct indexing here
    Kd = np.zeros((cfg.Hkv, n, cfg.d))
    Vd = np.zeros((cfg.Hkv, n, cfg.d))
    for p in range(n):
        pg = kv.block_table[0][p // cfg.page_size]
        Kd[:, p] = synth.bf16_bits_to_f32(kv.k[pg, :, p % cfg.page_size]).astype(np.float64)
        Vd[:, p] = synth.bf16_bits_to_f32(kv.v[pg, :, p % cfg.page_size]).astype(np.float64)
    Qt = torch.tensor(synth.bf16_bits_to_f32(q[0]).astype(np.float64)).permute(1, 0, 2)  # [Hq][n_q][d]
    Kt = torch.tensor(Kd).repeat_interleave(cfg.G, dim=0)
    Vt = torch.tensor(Vd).repeat_interleave(cfg.G, dim=0)
    mask = torch.zeros(cfg.n_q, n, dtype=torch.bool)
    for i in range(cfg.n_q):
        mask[i, :L + i + 1] = True
    ref = torch.nn.functional.scaled_dot_product_attention(
        Qt.unsqueeze(0), Kt.unsqueeze(0), Vt.unsqueeze(0), attn_mask=mask, scale=scale)[0]
    np.testing.assert_allclose(out[0], ref.permute(1, 0, 2).numpy(), rtol=0, atol=1e-12)
    lg = (Qt @ Kt.transpose(-1, -2)) * scale                 # [Hq][n_q][n]
    np.testing.assert_allclose(logits[0, :, 0, :L], lg[:, 0, :L].numpy(), atol=1e-12, rtol=0)
    np.testing.assert_allclose(logits[0, :, 1, :L], lg[:, cfg.n_q - 1, :L].numpy(), atol=1e-12, rtol=0)


def _set_rows(cache, block_table, b, g, positions, P, value_bits):
    for p in positions:
        cache[block_table[b][p // P], g, p % P, :] = value_bits


def test_closed_forms():
    cfg = small_cfg(B=1, L=30)
    kv, q = make(cfg, seed=2)
    scale = 1.0 / math.sqrt(cfg.d)
    n = cfg.L + cfg.n_q
    # K == 0: uniform weights, O = mean of the visible V rows
    k0 = kv.k.copy()
    k0[:] = 0
    out, _, lse = oa.verify_attn(q, k0, kv.v, kv.block_table, kv.prefix_len, cfg.page_size, scale)
    for g in range(cfg.Hkv):
        V = oa.paged_rows(kv.v, kv.block_table, 0, g, np.arange(n), cfg.page_size)
        for i in range(cfg.n_q):
            vis = cfg.L + i + 1
            for h in range(g * cfg.G, (g + 1) * cfg.G):
                np.testing.assert_allclose(out[0, i, h], V[:vis].mean(axis=0), atol=1e-12)
                assert abs(lse[0, i, h] - math.log(vis)) < 1e-12
    # V == 1: O == 1 exactly up to rounding
    v1 = kv.v.copy()
    v1[:] = 0x3F80  # bf16 1.0
    out, _, _ = oa.verify_attn(q, kv.k, v1, kv.block_table, kv.prefix_len, cfg.page_size, scale)
    np.testing.assert_allclose(out, 1.0, atol=1e-12)
    # one dominant key: q = e0 * 8 for every head, K[p*] = e0 * 100 -> logit 100 above others
    qd = np.zeros_like(q)
    qd[..., 0] = 0x4100  # bf16 8.0
    kd = np.zeros_like(kv.k)
    pstar = 11
    kd[kv.block_table[0][pstar // cfg.page_size], :, pstar % cfg.page_size, 0] = 0x4448  # 800.0
    out, logits, _ = oa.verify_attn(qd, kd, kv.v, kv.block_table, kv.prefix_len,
                                    cfg.page_size, 1.0 / 64.0)  # logit 8*800/64 = 100
    for g in range(cfg.Hkv):
        vrow = oa.paged_rows(kv.v, kv.block_table, 0, g, np.array([pstar]), cfg.page_size)[0]
        for h in range(g * cfg.G, (g + 1) * cfg.G):
            np.testing.assert_allclose(out[0, :, h], np.broadcast_to(vrow, (cfg.n_q, cfg.d)), atol=1e-30)
            assert logits[0, h, 0, pstar] == 100.0


def test_softmax_rows_sum_to_one():
    cfg = small_cfg()
    kv, q = make(cfg, seed=4, lens=[37, 9])
    _, _, _, W = oa.verify_attn(q, kv.k, kv.v, kv.block_table, kv.prefix_len, cfg.page_size,
                                0.25, return_weights=True)
    for (b, g), P in W.items():
        np.testing.assert_allclose(P.sum(axis=-1), 1.0, atol=1e-12)
        L = int(kv.prefix_len[b])
        for i in range(cfg.n_q):   # chain causality: nothing beyond slot i
            assert np.all(P[i, :, L + i + 1:] == 0)


def test_chain_equals_explicit_chain_mask():
    cfg = small_cfg()
    kv, q = make(cfg, seed=5)
    tm = np.stack([synth.chain_tail_masks(cfg.n_q)] * cfg.B)
    a = oa.verify_attn(q, kv.k, kv.v, kv.block_table, kv.prefix_len, cfg.page_size, 0.3)
    b = oa.verify_attn(q, kv.k, kv.v, kv.block_table, kv.prefix_len, cfg.page_size, 0.3, tree_mask=tm)
    for x, y in zip(a, b):
        np.testing.assert_array_equal(np.nan_to_num(x, nan=7.0), np.nan_to_num(y, nan=7.0))


def test_sparse_all_selected_equals_dense():
    cfg = small_cfg()
    kv, q = make(cfg, seed=6, lens=[37, 25])
    scale = 1.0 / math.sqrt(cfg.d)
    dense, _, dlse = oa.verify_attn(q, kv.k, kv.v, kv.block_table, kv.prefix_len, cfg.page_size, scale)
    cap = 64
    for mode in ("shared", "per_kv_head"):
        S = 1 if mode == "shared" else cfg.Hkv
        idx = np.full((cfg.B, S, cap), -1, dtype=np.int32)
        cnt = np.zeros((cfg.B, S), dtype=np.int32)
        for b in range(cfg.B):
            L = int(kv.prefix_len[b])
            idx[b, :, :L] = np.arange(L)
            cnt[b, :] = L
        tm = np.stack([synth.chain_tail_masks(cfg.n_q)] * cfg.B)
        out, lse = oa.sparse_attn(q, kv.k, kv.v, kv.block_table, cfg.page_size, mode, idx, cnt,
                                  kv.prefix_len, np.full(cfg.B, cfg.n_q), scale, tail_mask=tm)
        np.testing.assert_allclose(out, dense, atol=1e-12, rtol=0)
        np.testing.assert_allclose(lse, dlse, atol=1e-12, rtol=0)


def test_sparse_block_all_blocks_equals_dense_tree():
    cfg = small_cfg(B=1, L=37, page_size=8, n_q=4)   # last block is partial: clipped at L
    kv, q = make(cfg, seed=7)
    scale = 1.0 / math.sqrt(cfg.d)
    tm = np.stack([synth.tree_tail_masks(4, 2)])
    dense, _, _ = oa.verify_attn(q, kv.k, kv.v, kv.block_table, kv.prefix_len, cfg.page_size,
                                 scale, tree_mask=tm)
    nb = (cfg.L + cfg.page_size - 1) // cfg.page_size
    idx = np.tile(np.arange(nb, dtype=np.int32), (1, cfg.n_q, cfg.Hkv, 1))
    cnt = np.full((1, cfg.n_q, cfg.Hkv), nb, dtype=np.int32)
    out, _ = oa.sparse_attn(q, kv.k, kv.v, kv.block_table, cfg.page_size, "block", idx, cnt,
                            kv.prefix_len, np.array([cfg.n_q]), scale, tail_mask=tm)
    np.testing.assert_allclose(out, dense, atol=1e-12, rtol=0)


def test_sparse_block_matches_brute_force():
    cfg = small_cfg(B=1, L=64, page_size=8, n_q=4, Hq=4, Hkv=2)
    kv, q = make(cfg, seed=8)
    scale = 1.0 / math.sqrt(cfg.d)
    tm = np.stack([synth.tree_tail_masks(4, 2)])
    rng = np.random.default_rng(0)
    cap = 3
    idx = np.zeros((1, cfg.n_q, cfg.Hkv, cap), dtype=np.int32)
    for i in range(cfg.n_q):
        for g in range(cfg.Hkv):
            idx[0, i, g] = np.sort(rng.choice(8, size=cap, replace=False))
    cnt = np.full((1, cfg.n_q, cfg.Hkv), cap, dtype=np.int32)
    out, lse = oa.sparse_attn(q, kv.k, kv.v, kv.block_table, cfg.page_size, "block", idx, cnt,
                              kv.prefix_len, np.array([cfg.n_q]), scale, tail_mask=tm)
    for i in range(cfg.n_q):
        for h in range(cfg.Hq):
            g = h // cfg.G
            vis = [c * 8 + t for c in idx[0, i, g] for t in range(8)]
            vis += [cfg.L + j for j in range(cfg.n_q) if (int(tm[0][i]) >> j) & 1]
            o, l, _ = brute.attend(q[0, i, h], kv.k, kv.v, kv.block_table, 0, g, vis, 8, scale)
            np.testing.assert_allclose(out[0, i, h], o, atol=1e-12, rtol=0)
            assert abs(lse[0, i, h] - l) < 1e-12


def test_sparse_single_index_and_empty_list():
    cfg = small_cfg(B=1, n_q=1)
    kv, q = make(cfg, seed=9)
    scale = 1.0 / math.sqrt(cfg.d)
    idx = np.array([[[13]]], dtype=np.int32)
    cnt = np.array([[1]], dtype=np.int32)
    out, _ = oa.sparse_attn(q, kv.k, kv.v, kv.block_table, cfg.page_size, "shared", idx, cnt,
                            kv.prefix_len, np.array([0]), scale)
    for h in range(cfg.Hq):
        vrow = oa.paged_rows(kv.v, kv.block_table, 0, h // cfg.G, np.array([13]), cfg.page_size)[0]
        np.testing.assert_array_equal(out[0, 0, h], vrow)
    # empty list: attention over the tail only
    cnt0 = np.array([[0]], dtype=np.int32)
    out, lse = oa.sparse_attn(q, kv.k, kv.v, kv.block_table, cfg.page_size, "shared", idx, cnt0,
                              kv.prefix_len, np.array([3]), scale)
    for h in range(cfg.Hq):
        vis = [cfg.L + j for j in range(3)]
        o, l, _ = brute.attend(q[0, 0, h], kv.k, kv.v, kv.block_table, 0, h // cfg.G, vis,
                               cfg.page_size, scale)
        np.testing.assert_allclose(out[0, 0, h], o, atol=1e-12, rtol=0)
    # nothing visible at all: zero output, lse = -inf
    out, lse = oa.sparse_attn(q, kv.k, kv.v, kv.block_table, cfg.page_size, "shared", idx, cnt0,
                              kv.prefix_len, np.array([0]), scale)
    assert np.all(out == 0) and np.all(np.isneginf(lse))


def test_verify_any_row_set_matches_brute_force():
    """Collected rows in any order and count: slot c is row rows[c], against the
    scalar brute force."""
    cfg = small_cfg(n_q=5)
    kv, q = make(cfg, seed=4, lens=[29, 37])
    scale = 1.0 / math.sqrt(cfg.d)
    for rows in ([2], [4, 1, 3], list(range(5))):
        _, logits, _ = oa.verify_attn(q, kv.k, kv.v, kv.block_table, kv.prefix_len, cfg.page_size, scale,
                                      collect_rows=rows)
        assert logits.shape[2] == len(rows)
        for b in range(cfg.B):
            L = int(kv.prefix_len[b])
            for c, r in enumerate(rows):
                for h in range(cfg.Hq):
                    _, _, lg = brute.attend(q[b, r, h], kv.k, kv.v, kv.block_table, b, h // cfg.G,
                                            list(range(L + r + 1)), cfg.page_size, scale)
                    np.testing.assert_allclose(logits[b, h, c, :L], lg[:L], rtol=0, atol=1e-12)


def test_attention_one_matches_brute_and_verify_row():
    """attention_one (the checker of every sampled full-size comparison) against the
    scalar brute force on the same gathered rows, and against one row of verify_attn:
    output, weights and lse.  A dropped scale, an unshifted exponent or a wrong lse
    fails here."""
    cfg = small_cfg(B=1, n_q=3)
    kv, q = make(cfg, seed=12)
    scale = 1.0 / math.sqrt(cfg.d)
    out, _, lse, W = oa.verify_attn(q, kv.k, kv.v, kv.block_table, kv.prefix_len, cfg.page_size, scale,
                                    return_weights=True)
    L = cfg.L
    for i in range(cfg.n_q):
        vis = np.arange(L + i + 1)
        for h in range(cfg.Hq):
            g = h // cfg.G
            K = oa.paged_rows(kv.k, kv.block_table, 0, g, vis, cfg.page_size)
            V = oa.paged_rows(kv.v, kv.block_table, 0, g, vis, cfg.page_size)
            o, p, l = oa.attention_one(oa.bf16_to_f64(q[0, i, h]), K, V, scale)
            bo, bl, blg = brute.attend(q[0, i, h], kv.k, kv.v, kv.block_table, 0, g, vis.tolist(),
                                       cfg.page_size, scale)
            np.testing.assert_allclose(o, bo, rtol=0, atol=1e-12)
            assert abs(l - bl) < 1e-12
            # weights: exp(logit - lse) from the brute-force logits, summing to 1
            np.testing.assert_allclose(p, np.exp(np.asarray(blg) - bl), rtol=0, atol=1e-12)
            assert abs(p.sum() - 1.0) < 1e-12
            # and the same row of the dense verify
            np.testing.assert_allclose(o, out[0, i, h], rtol=0, atol=1e-12)
            assert abs(l - lse[0, i, h]) < 1e-12
            np.testing.assert_allclose(p, W[(0, g)][i, h - g * cfg.G, :L + i + 1], rtol=0, atol=1e-12)


def test_attention_one_scale_and_shift():
    """Closed forms: two keys whose logits differ by s give weights (1, e^-s)/(1 + e^-s);
    the lse is the larger logit plus log(1 + e^-s), whatever the common offset."""
    q = np.array([1.0, 0.0])
    K = np.array([[500.0, 0.0], [496.0, 0.0]])
    V = np.array([[1.0, 0.0], [0.0, 1.0]])
    o, p, l = oa.attention_one(q, K, V, 0.5)        # logits 250 and 248
    w = math.exp(-2.0)
    np.testing.assert_allclose(p, [1 / (1 + w), w / (1 + w)], rtol=1e-15)
    np.testing.assert_allclose(o, [1 / (1 + w), w / (1 + w)], rtol=1e-15)
    assert abs(l - (250.0 + math.log1p(w))) < 1e-12


def test_sparse_per_kv_head_distinct_lists_match_brute_force():
    """Per-KV-head sets with a different list for every KV head: head h must read the
    list of its own group h // G, not the first group's."""
    cfg = small_cfg(B=2, Hq=6, Hkv=3, L=40, n_q=2)
    kv, q = make(cfg, seed=13, lens=[40, 33])
    scale = 1.0 / math.sqrt(cfg.d)
    rng = np.random.default_rng(5)
    cap = 9
    idx = np.full((cfg.B, cfg.Hkv, cap), -1, dtype=np.int32)
    cnt = np.zeros((cfg.B, cfg.Hkv), dtype=np.int32)
    for b in range(cfg.B):
        L = int(kv.prefix_len[b])
        for g in range(cfg.Hkv):
            n = 3 + 2 * g                                       # every group a different size
            idx[b, g, :n] = np.sort(rng.choice(L, size=n, replace=False))
            cnt[b, g] = n
        assert len({tuple(idx[b, g, :cnt[b, g]]) for g in range(cfg.Hkv)}) == cfg.Hkv
    tl = np.array([2, 1], dtype=np.int32)
    out, lse = oa.sparse_attn(q, kv.k, kv.v, kv.block_table, cfg.page_size, "per_kv_head", idx, cnt,
                              kv.prefix_len, tl, scale)
    for b in range(cfg.B):
        tb = int(kv.prefix_len[b])
        for i in range(cfg.n_q):
            for h in range(cfg.Hq):
                g = h // cfg.G
                vis = idx[b, g, :cnt[b, g]].tolist() + [tb + j for j in range(int(tl[b]))]
                o, l, _ = brute.attend(q[b, i, h], kv.k, kv.v, kv.block_table, b, g, vis, cfg.page_size, scale)
                np.testing.assert_allclose(out[b, i, h], o, rtol=0, atol=1e-12)
                assert abs(lse[b, i, h] - l) < 1e-12
