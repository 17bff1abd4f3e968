"""Full-size parity at the 64K (per-KV-head, B=4, 40/8 heads) and 128K (B=8) workloads,
in the launch configurations the benchmark and the loop driver use, and for one 100K
sequence of the 8B-shaped layer with a 20K-entry set: there verify splits each KV head
96 ways, so the split-K merge loads its partials in three chunks, and the draft step
merges 32 splits.

The oracle cannot evaluate these calls whole, so it checks sampled outputs one by one:
for a sampled (sequence, row, head) it gathers the visible K/V rows itself and runs
plain fp64 softmax attention.  Selection is checked bit for bit with the pinned-order
CPU rule on the GPU's own logits, for a few sets, and the fused per-KV-head partial
scores bit for bit against the pinned sums of those logits.
"""
import numpy as np
import pytest

from long_context_self_amd import synth
from oracle import attention as oa
from oracle import select as osel

from gpu_helpers import bf16_dev, i32_dev, kv_dev, logit_rel_err, require_gpu, scale_for

pytestmark = pytest.mark.gpu

OUT_TOL = 1e-2
LOGIT_TOL = 1e-3


class Case:
    pass


# a single long sequence: more verify splits than one chunk of the merge's loads holds
LONG_SINGLE = synth.CONFIGS["llama8b_32k"].with_(name="llama8b_100k_b1", L=100000, top_k=20000)


def build(name):
    torch, lcs = require_gpu()
    c = Case()
    c.cfg = LONG_SINGLE if name == LONG_SINGLE.name else synth.CONFIGS[name]
    c.kv = synth.make_paged_kv(c.cfg, seed=0)
    c.q = synth.make_queries(c.cfg, c.kv, c.cfg.n_q, seed=0)
    c.qd = synth.make_queries(c.cfg, c.kv, 1, seed=0, tag=100)
    c.dkv = kv_dev(c.kv, torch, lcs)
    cfg = c.cfg
    B, L = cfg.B, cfg.L
    pl = i32_dev(c.kv.prefix_len, torch)
    out = torch.full((B, cfg.n_q, cfg.Hq, cfg.d), float("nan"), device="cuda")
    logits = torch.full((B, cfg.Hq, 2, L), float("nan"), device="cuda")
    lse = torch.full((B, cfg.n_q, cfg.Hq), float("nan"), device="cuda")
    lcs.verify_attn(c.dkv, bf16_dev(c.q, torch), pl, L, scale_for(cfg.d), cfg.collect_rows, out=out,
                    logits=logits, lse=lse)
    n_sets = 1 if cfg.mode == "shared" else cfg.Hkv
    S = cfg.n_sink + cfg.top_k + cfg.n_recent
    idx = torch.full((B, n_sets, S), -1, dtype=torch.int32, device="cuda")
    cnt = torch.zeros((B, n_sets), dtype=torch.int32, device="cuda")
    lcs.select_topk(logits, pl, L, cfg.Hkv, cfg.mode, cfg.top_k, cfg.n_sink, cfg.n_recent, cap=S,
                    indices=idx, counts=cnt)
    tl = np.full(B, cfg.n_q + 1, dtype=np.int32)
    dout = torch.full((B, 1, cfg.Hq, cfg.d), float("nan"), device="cuda")
    dlse = torch.full((B, 1, cfg.Hq), float("nan"), device="cuda")
    lcs.sparse_draft_attn(c.dkv, bf16_dev(c.qd, torch), cfg.mode, idx, cnt, pl, i32_dev(tl, torch),
                          cfg.n_q + cfg.n_draft, scale_for(cfg.d), out=dout, lse=dlse)
    scores = torch.full((B, cfg.Hkv, L), float("nan"), device="cuda")
    lcs.verify_attn_scores(c.dkv, bf16_dev(c.q, torch), pl, L, scale_for(cfg.d), cfg.collect_rows,
                           scores=scores)
    # the physical-slot hand-off on the same logits (the bench's physical_hand_off variant)
    pidx = torch.full((B, n_sets, S), -1, dtype=torch.int32, device="cuda")
    pcnt = torch.zeros((B, n_sets), dtype=torch.int32, device="cuda")
    lcs.select_topk_physical(logits, pl, L, cfg.Hkv, cfg.mode, cfg.top_k, cfg.n_sink, cfg.n_recent, c.dkv,
                             cap=S, indices=pidx, counts=pcnt)
    pdout = torch.full((B, 1, cfg.Hq, cfg.d), float("nan"), device="cuda")
    pdlse = torch.full((B, 1, cfg.Hq), float("nan"), device="cuda")
    lcs.sparse_draft_attn_physical(c.dkv, bf16_dev(c.qd, torch), cfg.mode, pidx, pcnt, pl, i32_dev(tl, torch),
                                   cfg.n_q + cfg.n_draft, scale_for(cfg.d), out=pdout, lse=pdlse)
    torch.cuda.synchronize()
    c.scores = scores.cpu().numpy()
    c.pidx, c.pcnt = pidx.cpu().numpy(), pcnt.cpu().numpy()
    c.pdout, c.pdlse = pdout.cpu().numpy(), pdlse.cpu().numpy()
    c.out, c.logits, c.lse = out.cpu().numpy(), logits.cpu().numpy(), lse.cpu().numpy()
    c.idx, c.cnt, c.tl = idx.cpu().numpy(), cnt.cpu().numpy(), tl
    c.dout, c.dlse = dout.cpu().numpy(), dlse.cpu().numpy()
    del c.dkv
    torch.cuda.empty_cache()
    return c


@pytest.fixture(scope="module", params=["qwen14b_64k", "stress_128k", LONG_SINGLE.name])
def case(request):
    return build(request.param)


def test_verify_sampled(case):
    cfg, kv = case.cfg, case.kv
    sc = scale_for(cfg.d)
    qf = oa.bf16_to_f64(case.q)
    rng = np.random.default_rng(1)
    assert np.isfinite(case.out).all()
    for _ in range(10):
        b, i, h = int(rng.integers(cfg.B)), int(rng.integers(cfg.n_q)), int(rng.integers(cfg.Hq))
        g, L = h // cfg.G, int(kv.prefix_len[b])
        pos = np.arange(L + i + 1)
        K = oa.paged_rows(kv.k, kv.block_table, b, g, pos, cfg.page_size)
        V = oa.paged_rows(kv.v, kv.block_table, b, g, pos, cfg.page_size)
        o, _, l = oa.attention_one(qf[b, i, h], K, V, sc)
        assert np.max(np.abs(case.out[b, i, h] - o)) <= OUT_TOL
        assert abs(case.lse[b, i, h] - l) <= 1e-3
    for _ in range(4):                 # whole collected logit rows
        b, h, c = int(rng.integers(cfg.B)), int(rng.integers(cfg.Hq)), int(rng.integers(2))
        i = 0 if c == 0 else cfg.n_q - 1
        L = int(kv.prefix_len[b])
        K = oa.paged_rows(kv.k, kv.block_table, b, h // cfg.G, np.arange(L), cfg.page_size)
        assert logit_rel_err(case.logits[b, h, c, :L], sc * (K @ qf[b, i, h])) <= LOGIT_TOL


def test_select_exact_on_gpu_logits(case):
    cfg = case.cfg
    rng = np.random.default_rng(2)
    n_sets = 1 if cfg.mode == "shared" else cfg.Hkv
    for _ in range(3):
        b, s = int(rng.integers(cfg.B)), int(rng.integers(n_sets))
        L = int(case.kv.prefix_len[b])
        heads = range(cfg.Hq) if cfg.mode == "shared" else range(s * cfg.G, (s + 1) * cfg.G)
        ref = osel.topk_tokens(osel.scores_f32_pinned(case.logits, b, L, heads), L, cfg.top_k, cfg.n_sink,
                               cfg.n_recent)
        assert case.cnt[b, s] == ref.size
        assert np.array_equal(case.idx[b, s, :ref.size], ref)


def test_draft_sampled(case):
    cfg, kv = case.cfg, case.kv
    sc = scale_for(cfg.d)
    qf = oa.bf16_to_f64(case.qd)
    rng = np.random.default_rng(3)
    assert np.isfinite(case.dout).all()
    for _ in range(10):
        b, h = int(rng.integers(cfg.B)), int(rng.integers(cfg.Hq))
        g, L = h // cfg.G, int(kv.prefix_len[b])
        sel = oa.sparse_visible_positions(cfg.mode, case.idx, case.cnt, b, 0, g, cfg.page_size, L)
        pos = np.concatenate([sel, L + np.arange(int(case.tl[b]))])
        K = oa.paged_rows(kv.k, kv.block_table, b, g, pos, cfg.page_size)
        V = oa.paged_rows(kv.v, kv.block_table, b, g, pos, cfg.page_size)
        o, _, l = oa.attention_one(qf[b, 0, h], K, V, sc)
        assert np.max(np.abs(case.dout[b, 0, h] - o)) <= OUT_TOL
        assert abs(case.dlse[b, 0, h] - l) <= 1e-3


def test_partial_scores_bit_exact(case):
    """The fused partial scores equal the pinned CPU sums of the written logits."""
    cfg = case.cfg
    for b in range(cfg.B):
        L = int(case.kv.prefix_len[b])
        want = osel.partial_scores_f32(case.logits, b, L, cfg.Hq, cfg.Hkv)
        assert np.array_equal(case.scores[b, :, :L].view(np.uint32), want.view(np.uint32)), f"b {b}"


def test_long_tree_two_row_chunks_sampled():
    """128K prefix, 16 verifier rows (64 q-rows per KV group: two row chunks, whose launch
    loads K/V with caching so that the chunks' re-reads hit), logit rows at the padded
    stride: sampled rows of both chunks and both collected rows against the oracle."""
    torch, lcs = require_gpu()
    cfg = synth.CONFIGS["stress_128k"].with_(B=2, n_q=16)
    kv = synth.make_paged_kv(cfg, seed=7)
    q = synth.make_queries(cfg, kv, cfg.n_q, seed=7)
    dkv = kv_dev(kv, torch, lcs)
    B, L = cfg.B, cfg.L
    ld = lcs.row_ld(L)
    out = torch.full((B, cfg.n_q, cfg.Hq, cfg.d), float("nan"), device="cuda")
    logits = torch.full((B, cfg.Hq, 2, ld), float("nan"), device="cuda")
    lse = torch.full((B, cfg.n_q, cfg.Hq), float("nan"), device="cuda")
    lcs.verify_attn(dkv, bf16_dev(q, torch), i32_dev(kv.prefix_len, torch), L, scale_for(cfg.d),
                    (0, cfg.n_q - 1), out=out, logits=logits, lse=lse)
    torch.cuda.synchronize()
    out, logits, lse = out.cpu().numpy(), logits.cpu().numpy(), lse.cpu().numpy()
    del dkv
    torch.cuda.empty_cache()
    assert np.isfinite(out).all()
    sc = scale_for(cfg.d)
    qf = oa.bf16_to_f64(q)
    rng = np.random.default_rng(4)
    for i in (0, 5, 11, 12, 15, int(rng.integers(cfg.n_q))):   # rows 0-11: chunk 0, 12-15: chunk 1
        b, h = int(rng.integers(B)), int(rng.integers(cfg.Hq))
        g, Lb = h // cfg.G, int(kv.prefix_len[b])
        pos = np.arange(Lb + i + 1)
        K = oa.paged_rows(kv.k, kv.block_table, b, g, pos, cfg.page_size)
        V = oa.paged_rows(kv.v, kv.block_table, b, g, pos, cfg.page_size)
        o, _, l = oa.attention_one(qf[b, i, h], K, V, sc)
        assert np.max(np.abs(out[b, i, h] - o)) <= OUT_TOL, f"row {i}"
        assert abs(lse[b, i, h] - l) <= 1e-3
    for c, i in ((0, 0), (1, cfg.n_q - 1)):
        b, h = int(rng.integers(B)), int(rng.integers(cfg.Hq))
        Lb = int(kv.prefix_len[b])
        K = oa.paged_rows(kv.k, kv.block_table, b, h // cfg.G, np.arange(Lb), cfg.page_size)
        assert logit_rel_err(logits[b, h, c, :Lb], sc * (K @ qf[b, i, h])) <= LOGIT_TOL
        assert np.isnan(logits[b, h, c, Lb:]).all()


def test_physical_hand_off_full(case):
    """Select's physical slots are its logical selection mapped through the block table
    (slot = page << log2(page size) | offset), and the draft over them equals the draft
    over the positions bit for bit, at the full workload."""
    cfg, kv = case.cfg, case.kv
    lg = int(cfg.page_size).bit_length() - 1
    assert np.array_equal(case.pcnt, case.cnt)
    for b in range(cfg.B):
        for s in range(case.cnt.shape[1]):
            n = int(case.cnt[b, s])
            pos = case.idx[b, s, :n].astype(np.int64)
            want = (kv.block_table[b, pos >> lg].astype(np.int64) << lg) | (pos & (cfg.page_size - 1))
            assert np.array_equal(case.pidx[b, s, :n].astype(np.int64), want), f"b {b} set {s}"
    assert np.array_equal(case.pdout.view(np.uint32), case.dout.view(np.uint32))
    assert np.array_equal(case.pdlse.view(np.uint32), case.dlse.view(np.uint32))


def test_select_from_partial_scores_full(case):
    """Select from the fused per-KV-head partial scores at the full workload (the launch
    that sums one row per KV head, several 512-position chunks per workgroup) equals the
    CPU rule on those scores bit for bit; with per-KV-head sets it also equals the
    selection from the logit rows."""
    torch, lcs = require_gpu()
    cfg = case.cfg
    S = cfg.n_sink + cfg.top_k + cfg.n_recent
    sc = torch.from_numpy(np.ascontiguousarray(case.scores)).cuda()
    pl = i32_dev(case.kv.prefix_len, torch)
    idx, cnt = lcs.select_topk_scores(sc, pl, cfg.L, cfg.mode, cfg.top_k, cfg.n_sink, cfg.n_recent, cap=S,
                                      Hq=cfg.Hq)
    torch.cuda.synchronize()
    gi, gc = idx.cpu().numpy(), cnt.cpu().numpy()
    ref = osel.select(case.scores[:, :, None, :], case.kv.prefix_len, cfg.Hkv, cfg.mode, cfg.top_k, cfg.n_sink,
                      cfg.n_recent, precision="f32")
    for b in range(cfg.B):
        for s, r in enumerate(ref[b]):
            assert gc[b, s] == r.size and np.array_equal(gi[b, s, :r.size], r), f"b {b} set {s}"
    if cfg.mode == "per_kv_head":
        assert np.array_equal(gc, case.cnt) and np.array_equal(gi, case.idx)
