"""Calls on two streams at once, each with its own workspace and outputs, give exactly
what the same calls give one after the other: the library keeps no state between calls
besides the workspaces the caller passes (the no-allocation draft call aside)."""
import numpy as np
import pytest

from long_context_self_amd import synth

from gpu_helpers import bf16_dev, i32_dev, kv_dev, require_gpu, scale_for

pytestmark = pytest.mark.gpu


def test_two_streams_match_sequential():
    torch, lcs = require_gpu()
    cfg = synth.CONFIGS["llama8b_32k"].with_(L=4096, B=2)
    kv = synth.make_paged_kv(cfg, seed=11)
    dkv = kv_dev(kv, torch, lcs)
    pl = i32_dev(kv.prefix_len, torch)
    L = int(kv.prefix_len.max())
    qs = [bf16_dev(synth.make_queries(cfg, kv, cfg.n_q, seed=20 + i), torch) for i in range(2)]
    S = cfg.n_sink + cfg.top_k + cfg.n_recent
    tl = i32_dev(np.full(cfg.B, cfg.n_q + 1, dtype=np.int32), torch)
    qd = bf16_dev(synth.make_queries(cfg, kv, 1, seed=30), torch)

    def run(q):
        _, lg, _ = lcs.verify_attn(dkv, q, pl, L, scale_for(cfg.d), cfg.collect_rows)
        idx, cnt = lcs.select_topk(lg, pl, L, cfg.Hkv, cfg.mode, cfg.top_k, cfg.n_sink, cfg.n_recent, cap=S)
        out, _ = lcs.sparse_draft_attn(dkv, qd, cfg.mode, idx, cnt, pl, tl, cfg.n_q + 1, scale_for(cfg.d))
        return lg, idx, cnt, out

    seq = [run(q) for q in qs]
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for st in streams:
        st.wait_stream(torch.cuda.current_stream())
    par = [None, None]
    for rep in range(3):
        for i, st in enumerate(streams):
            with torch.cuda.stream(st):
                par[i] = run(qs[i])
        torch.cuda.synchronize()
        for i in range(2):
            for a, b in zip(seq[i], par[i]):
                assert torch.equal(a, b), f"stream {i}, repeat {rep}"
