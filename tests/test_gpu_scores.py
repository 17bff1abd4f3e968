"""GPU parity of the per-KV-head partial scores (lcs_verify_attn_scores) and of
selection from them (lcs_select_topk_scores).

The verify kernel's scaled logits are the same bits in both verify entry points, so
the partial scores must equal, bit for bit, the pinned-order CPU sum of the logits
that lcs_verify_attn writes for the same inputs; selection from them must equal the
CPU rule on those partials, and for per-KV-head and block sets the selection on the
logits themselves.
"""
import numpy as np
import pytest

from long_context_self_amd import synth
from oracle import select as osel

from gpu_helpers import bf16_dev, i32_dev, kv_dev, require_gpu, scale_for

pytestmark = pytest.mark.gpu


def run(cfg, seed, lens=None, rows=None):
    torch, lcs = require_gpu()
    kv = synth.make_paged_kv(cfg, seed=seed, lens=lens)
    q = synth.make_queries(cfg, kv, cfg.n_q, seed=seed)
    dkv, dq, pl = kv_dev(kv, torch, lcs), bf16_dev(q, torch), i32_dev(kv.prefix_len, torch)
    maxL = int(kv.prefix_len.max())
    rows = rows or (0, cfg.n_q - 1)
    out1, lg, lse1 = lcs.verify_attn(dkv, dq, pl, maxL, scale_for(cfg.d), rows)
    sc = torch.full((cfg.B, cfg.Hkv, maxL + 3), float("nan"), device="cuda")
    out2, _, lse2 = lcs.verify_attn_scores(dkv, dq, pl, maxL, scale_for(cfg.d), rows, scores=sc)
    torch.cuda.synchronize()
    assert torch.equal(out1, out2) and torch.equal(lse1, lse2)
    return torch, lcs, kv, pl, maxL, lg, sc


@pytest.mark.parametrize("name,L,B,rows", [("llama8b_32k", 3000, 2, None), ("qwen14b_64k", 2500, 2, None),
                                           ("tiny", 1024, 1, (3, 1)), ("tiny", 1024, 1, (2, 2))])
def test_partial_scores_bit_exact(name, L, B, rows):
    cfg = synth.CONFIGS[name].with_(L=L, B=B)
    lens = [L - 53 * b for b in range(B)]
    torch, lcs, kv, pl, maxL, lg, sc = run(cfg, 12, lens=lens, rows=rows)
    g_lg, g_sc = lg.cpu().numpy(), sc.cpu().numpy()
    for b in range(cfg.B):
        Lb = int(kv.prefix_len[b])
        want = osel.partial_scores_f32(g_lg, b, Lb, cfg.Hq, cfg.Hkv)
        assert np.array_equal(g_sc[b, :, :Lb].view(np.uint32), want.view(np.uint32)), f"b {b}"
        assert np.isnan(g_sc[b, :, Lb:]).all(), "columns past the prefix were written"


@pytest.mark.parametrize("mode", ["shared", "per_kv_head", "block"])
def test_select_from_scores(mode):
    cfg = synth.CONFIGS["llama8b_32k"].with_(L=6000, B=2, top_k=700)
    torch, lcs, kv, pl, maxL, lg, sc = run(cfg, 13, lens=[6000, 4999])
    bs = 64 if mode == "block" else 0
    k = 20 if mode == "block" else cfg.top_k
    sc = sc[:, :, :maxL].contiguous()
    idx, cnt = lcs.select_topk_scores(sc, pl, maxL, mode, k, cfg.n_sink, cfg.n_recent, block_size=bs, Hq=cfg.Hq)
    torch.cuda.synchronize()
    g_sc = sc.cpu().numpy()
    ref = osel.select(g_sc[:, :, None, :], kv.prefix_len, cfg.Hkv, mode, k, cfg.n_sink, cfg.n_recent,
                      block_size=bs, precision="f32")
    gi, gc = idx.cpu().numpy(), cnt.cpu().numpy()
    for b in range(cfg.B):
        for s, r in enumerate(ref[b]):
            assert gc[b, s] == r.size and np.array_equal(gi[b, s, :r.size], r), f"{mode} b{b} s{s}"
    if mode != "shared":
        i2, c2 = lcs.select_topk(lg, pl, maxL, cfg.Hkv, mode, k, cfg.n_sink, cfg.n_recent, block_size=bs)
        torch.cuda.synchronize()
        assert torch.equal(c2, cnt) and torch.equal(i2, idx)
