"""GPU parity of the row-set collection (lcs_verify_attn_rows) and of selection over
n collected rows, by summed logits and by softmax weights (lcs_select_topk_rows).

* Collected logits against the fp64 oracle within 1e-3 relative (as for the two
  rows); outputs and lse bit-identical to the two-row entry point, which runs the
  same kernel with another store pattern.
* Logit-sum selection over n rows: bit-exact against the pinned-order CPU rule on
  the GPU's own logits; n = 2 equals lcs_select_topk bit for bit.
* Softmax-weight selection: expf differs from numpy's exp by rounding, so the
  result is checked for validity against the fp64 score of the same GPU logits and
  lse: every kept pool item scores at least the k-th score minus eps, every dropped
  one at most the k-th plus eps, eps = 1e-5 relative (float32 sums of at most a few
  hundred positive terms, each within a few ulp), and the overlap with the fp64
  choice is at least 99 %.
"""
import numpy as np
import pytest

from long_context_self_amd import synth
from oracle import attention as oa
from oracle import select as osel

from gpu_helpers import bf16_dev, i32_dev, kv_dev, logit_rel_err, require_gpu, scale_for

pytestmark = pytest.mark.gpu

LOGIT_TOL = 1e-3
W_EPS = 1e-5


def setup(cfg, seed, lens=None):
    torch, lcs = require_gpu()
    kv = synth.make_paged_kv(cfg, seed=seed, lens=lens)
    q = synth.make_queries(cfg, kv, cfg.n_q, seed=seed)
    return torch, lcs, kv, q, kv_dev(kv, torch, lcs), bf16_dev(q, torch), i32_dev(kv.prefix_len, torch)


@pytest.mark.parametrize("rows", [[2], [4, 0, 2], "all"])
def test_verify_rows_against_oracle(rows):
    cfg = synth.CONFIGS["llama8b_32k"].with_(L=1500, B=2)
    torch, lcs, kv, q, dkv, dq, pl = setup(cfg, 7, lens=[1500, 1211])
    rows = list(range(cfg.n_q)) if rows == "all" else rows
    maxL = int(kv.prefix_len.max())
    out, lg, lse = lcs.verify_attn_rows(dkv, dq, pl, maxL, scale_for(cfg.d), rows)
    out2, lg2, lse2 = lcs.verify_attn(dkv, dq, pl, maxL, scale_for(cfg.d), (0, cfg.n_q - 1))
    torch.cuda.synchronize()
    assert torch.equal(out, out2) and torch.equal(lse, lse2)
    srt = sorted(rows)
    _, o_lg, _ = oa.verify_attn(q, kv.k, kv.v, kv.block_table, kv.prefix_len, cfg.page_size, scale_for(cfg.d),
                                collect_rows=srt)
    g = lg.cpu().numpy()
    assert g.shape[2] == len(rows)
    for b in range(cfg.B):
        L = int(kv.prefix_len[b])
        e = logit_rel_err(g[b, :, :, :L], o_lg[b, :, :, :L])
        assert e <= LOGIT_TOL, f"rows {rows} b {b}: logit rel err {e}"
    # the two-row layout through the mask entry point is the Collect-2-Query layout
    if srt == [0, cfg.n_q - 1]:
        assert torch.equal(lg, lg2)


def test_verify_two_row_order_and_repeat():
    """The two-row entry point keeps its slot order (row0 to slot 0) when row0 > row1,
    and writes one row to both slots when they are equal."""
    cfg = synth.CONFIGS["tiny"]
    torch, lcs, kv, q, dkv, dq, pl = setup(cfg, 3)
    L = cfg.L
    n = cfg.n_q
    _, fwd, _ = lcs.verify_attn(dkv, dq, pl, L, scale_for(cfg.d), (0, n - 1))
    _, rev, _ = lcs.verify_attn(dkv, dq, pl, L, scale_for(cfg.d), (n - 1, 0))
    _, dup, _ = lcs.verify_attn(dkv, dq, pl, L, scale_for(cfg.d), (2, 2))
    _, one, _ = lcs.verify_attn_rows(dkv, dq, pl, L, scale_for(cfg.d), [2])
    torch.cuda.synchronize()
    assert torch.equal(rev[:, :, 0], fwd[:, :, 1]) and torch.equal(rev[:, :, 1], fwd[:, :, 0])
    assert torch.equal(dup[:, :, 0], one[:, :, 0]) and torch.equal(dup[:, :, 1], one[:, :, 0])


@pytest.mark.parametrize("mode", ["shared", "per_kv_head", "block"])
def test_select_logit_sum_n_rows_bit_exact(mode):
    cfg = synth.CONFIGS["llama8b_32k"].with_(L=6000, B=2, top_k=700)
    torch, lcs, kv, q, dkv, dq, pl = setup(cfg, 8, lens=[6000, 4321])
    maxL = int(kv.prefix_len.max())
    rows = list(range(cfg.n_q))
    _, lg, _ = lcs.verify_attn_rows(dkv, dq, pl, maxL, scale_for(cfg.d), rows)
    bs = 64 if mode == "block" else 0
    k = 20 if mode == "block" else cfg.top_k
    idx, cnt = lcs.select_topk_rows(lg, pl, maxL, cfg.Hkv, mode, k, cfg.n_sink, cfg.n_recent, block_size=bs)
    torch.cuda.synchronize()
    ref = osel.select(lg.cpu().numpy(), kv.prefix_len, cfg.Hkv, mode, k, cfg.n_sink, cfg.n_recent,
                      block_size=bs, precision="f32")
    gi, gc = idx.cpu().numpy(), cnt.cpu().numpy()
    for b in range(cfg.B):
        for s, r in enumerate(ref[b]):
            assert gc[b, s] == r.size
            assert np.array_equal(gi[b, s, :r.size], r), f"{mode} b{b} s{s}"


@pytest.mark.parametrize("row", [0, 8])
def test_select_single_row_bit_exact(row):
    """One collected row: the head sum of that row's logits, bit-exact."""
    cfg = synth.CONFIGS["llama8b_32k"].with_(L=5000, B=1, top_k=500)
    torch, lcs, kv, q, dkv, dq, pl = setup(cfg, 14)
    _, lg, _ = lcs.verify_attn_rows(dkv, dq, pl, cfg.L, scale_for(cfg.d), [row])
    idx, cnt = lcs.select_topk_rows(lg, pl, cfg.L, cfg.Hkv, "shared", cfg.top_k, cfg.n_sink, cfg.n_recent)
    torch.cuda.synchronize()
    ref = osel.select(lg.cpu().numpy(), kv.prefix_len, cfg.Hkv, "shared", cfg.top_k, cfg.n_sink, cfg.n_recent,
                      precision="f32")[0][0]
    assert cnt.cpu().numpy()[0, 0] == ref.size
    assert np.array_equal(idx.cpu().numpy()[0, 0, :ref.size], ref)


def test_select_rows_two_equals_select_topk():
    cfg = synth.CONFIGS["llama8b_32k"].with_(L=5000, B=1, top_k=600)
    torch, lcs, kv, q, dkv, dq, pl = setup(cfg, 9)
    _, lg, _ = lcs.verify_attn(dkv, dq, pl, cfg.L, scale_for(cfg.d), (0, cfg.n_q - 1))
    for mode in ("shared", "per_kv_head"):
        i1, c1 = lcs.select_topk(lg, pl, cfg.L, cfg.Hkv, mode, cfg.top_k, cfg.n_sink, cfg.n_recent)
        i2, c2 = lcs.select_topk_rows(lg, pl, cfg.L, cfg.Hkv, mode, cfg.top_k, cfg.n_sink, cfg.n_recent)
        torch.cuda.synchronize()
        assert torch.equal(c1, c2) and torch.equal(i1, i2)


@pytest.mark.parametrize("mode,rows", [("shared", [5, 6, 7, 8]), ("per_kv_head", "all"), ("block", [0, 8])])
def test_select_softmax_weights_valid(mode, rows):
    cfg = synth.CONFIGS["llama8b_32k"].with_(L=7000, B=2, top_k=800)
    torch, lcs, kv, q, dkv, dq, pl = setup(cfg, 10, lens=[7000, 5555])
    maxL = int(kv.prefix_len.max())
    rows = list(range(cfg.n_q)) if rows == "all" else rows
    _, lg, lse = lcs.verify_attn_rows(dkv, dq, pl, maxL, scale_for(cfg.d), rows)
    bs = 64 if mode == "block" else 0
    k = 25 if mode == "block" else cfg.top_k
    idx, cnt = lcs.select_topk_rows(lg, pl, maxL, cfg.Hkv, mode, k, cfg.n_sink, cfg.n_recent, score="weights",
                                    lse=lse, rows=rows, block_size=bs)
    torch.cuda.synchronize()
    g_lg, g_lse = lg.cpu().numpy(), lse.cpu().numpy()
    gi, gc = idx.cpu().numpy(), cnt.cpu().numpy()
    ref = osel.select(g_lg, kv.prefix_len, cfg.Hkv, mode, k, cfg.n_sink, cfg.n_recent, block_size=bs,
                      score_kind="weights", lse=g_lse, rows=rows)
    smode = "per_kv_head" if mode == "block" else mode
    for b in range(cfg.B):
        L = int(kv.prefix_len[b])
        for s, r in enumerate(ref[b]):
            assert gc[b, s] == r.size
            got = gi[b, s, :r.size].astype(np.int64)
            assert np.all(np.diff(got) > 0)
            heads = osel.set_heads(smode, cfg.Hq, cfg.Hkv, s)
            sig = osel.scores_weights_f64(g_lg, g_lse, rows, b, L, heads)
            if mode == "block":
                sig = osel.block_scores(sig, L, bs)
                nb, lo, hi = osel.block_window(L, bs, cfg.n_sink, cfg.n_recent)
            else:
                lo, hi = cfg.n_sink, L - cfg.n_recent
            pool = np.arange(lo, hi)
            kth = np.sort(sig[lo:hi])[::-1][k - 1]
            eps = W_EPS * max(kth, 1e-30)
            kept = np.isin(pool, got)
            assert np.all(sig[pool[kept]] >= kth - eps)
            assert np.all(sig[pool[~kept]] <= kth + eps)
            assert np.isin(r, got).mean() >= 0.99


@pytest.mark.parametrize("G", [1, 4])
def test_collect_all_64_rows(G):
    """The most verifier rows a call takes (n_q = 64), every one collected: the row mask
    uses all 64 bits and slot 63 is the last; logits of every row against the fp64
    oracle, outputs equal to those of the two-row call, and selection over the 64 rows'
    summed logits bit-exact against the pinned-order CPU rule.  G = 4 splits the 256
    q-rows of a KV head over six row chunks."""
    Hkv = 2
    cfg = synth.Config("rows64", B=2, Hq=G * Hkv, Hkv=Hkv, d=64, L=700, page_size=16, n_q=64, n_draft=0,
                       top_k=64, n_sink=4, n_recent=16, mode="shared", crit_frac=0.01)
    torch, lcs, kv, q, dkv, dq, pl = setup(cfg, 9, lens=[700, 333])
    rows = list(range(64))
    out, lg, lse = lcs.verify_attn_rows(dkv, dq, pl, 700, scale_for(cfg.d), rows)
    out2, _, lse2 = lcs.verify_attn(dkv, dq, pl, 700, scale_for(cfg.d), (0, 63))
    torch.cuda.synchronize()
    assert torch.equal(out, out2) and torch.equal(lse, lse2)
    _, o_lg, _ = oa.verify_attn(q, kv.k, kv.v, kv.block_table, kv.prefix_len, cfg.page_size, scale_for(cfg.d),
                                collect_rows=rows)
    g = lg.cpu().numpy()
    assert g.shape[2] == 64
    for b in range(cfg.B):
        L = int(kv.prefix_len[b])
        e = logit_rel_err(g[b, :, :, :L], o_lg[b, :, :, :L])
        assert e <= LOGIT_TOL, f"b {b}: logit rel err {e}"
    # selection over all 64 rows by their summed logits, in the pinned row order
    for mode in ("shared", "per_kv_head"):
        idx, cnt = lcs.select_topk_rows(lg, pl, 700, cfg.Hkv, mode, cfg.top_k, cfg.n_sink, cfg.n_recent)
        torch.cuda.synchronize()
        ref = osel.select(g, kv.prefix_len, cfg.Hkv, mode, cfg.top_k, cfg.n_sink, cfg.n_recent, precision="f32")
        gi, gc = idx.cpu().numpy(), cnt.cpu().numpy()
        for b in range(cfg.B):
            for s_, r in enumerate(ref[b]):
                assert gc[b, s_] == r.size and np.array_equal(gi[b, s_, :r.size], r), f"{mode} b{b} s{s_}"
