"""Speculative-iteration driver over the verify / select / draft calls.

One iteration of one layer follows the Vegas page ("The pith"): verify the n_q = k + 1
rows over the whole cache with the two collected logit rows, select the next sparse
set from those rows, then run k single-token draft steps over the set plus the tail
written since the selection.  Between iterations a fraction of the planted critical
positions moves (their K rows are redrawn), so the selection has something to track.

This is host orchestration only: every step of the path runs in the library's
kernels.  Per-call times come from HIP events on the calling stream; the recall of
the current critical positions in the selected set is a quality sanity check of the
synthetic workload, not a parity check.

    python -m long_context_self_amd.driver --config stress_128k --iters 256 [--scores]
"""
from __future__ import annotations

import argparse
import json
import math
import sys
import time

import numpy as np


def _bf16(torch, a, dev):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)


def recall(cfg, kv, idx: np.ndarray, cnt: np.ndarray) -> float:
    """Mean over (b, g) of the fraction of g's critical positions in the selected set."""
    vals = []
    for b in range(cfg.B):
        for g in range(cfg.Hkv):
            crit = kv.critical[b][g]
            if crit.size == 0:
                continue
            s = 0 if cfg.mode == "shared" else g
            sel = idx[b, s, :int(cnt[b, s])]
            vals.append(np.isin(crit, sel).mean())
    return float(np.mean(vals)) if vals else float("nan")


def run(cfg, iters: int, drift: float = 0.1, seed: int = 0, warmup: int = 1, log=None,
        scores: bool = False, keep_last: bool = False) -> dict:
    """scores: verify writes per-KV-head partial scores and select reads them, instead
    of the two collected logit rows (same selection rule, one row per KV head).

    keep_last: also return, under "last", host copies of the last iteration's inputs and
    outputs as the calls saw them (the K cache before that iteration's drift, the
    verifier and draft queries, verify's out and collected rows, the selected sets, the
    last draft step's output and tail length) and, after the final drift, the device K
    cache and the host cache it must equal."""
    import torch

    from . import lcs, synth

    assert cfg.mode in ("shared", "per_kv_head"), "the loop drives token-set selection"
    dev = "cuda"
    scale = 1.0 / math.sqrt(cfg.d)
    kv = synth.make_paged_kv(cfg, seed=seed)
    k_dev, v_dev = _bf16(torch, kv.k, dev), _bf16(torch, kv.v, dev)
    layer = lcs.PagedKV(k_dev, v_dev, torch.from_numpy(kv.block_table).to(dev))
    B, Hq, L, d = cfg.B, cfg.Hq, cfg.L, cfg.d
    n_sets = 1 if cfg.mode == "shared" else cfg.Hkv
    S = cfg.n_sink + cfg.top_k + cfg.n_recent
    pl = torch.from_numpy(kv.prefix_len).to(dev)
    if scores:
        logits = torch.empty((B, cfg.Hkv, lcs.row_ld(L)), dtype=torch.float32, device=dev)
    else:
        logits = torch.empty((B, Hq, 2, lcs.row_ld(L)), dtype=torch.float32, device=dev)
    out = torch.empty((B, cfg.n_q, Hq, d), dtype=torch.float32, device=dev)
    dout = torch.empty((B, 1, Hq, d), dtype=torch.float32, device=dev)
    idx = torch.empty((B, n_sets, S), dtype=torch.int32, device=dev)
    cnt = torch.empty((B, n_sets), dtype=torch.int32, device=dev)
    tls = [torch.full((B,), cfg.n_q + j + 1, dtype=torch.int32, device=dev) for j in range(cfg.n_draft)]
    max_tl = cfg.n_q + cfg.n_draft
    ws_v = torch.empty(lcs.verify_workspace_bytes(layer, B, cfg.n_q, Hq, L), dtype=torch.uint8, device=dev)
    ws_s = torch.empty(lcs.select_workspace_bytes(B, Hq, cfg.Hkv, cfg.mode, L), dtype=torch.uint8, device=dev)
    ws_d = torch.empty(lcs.sparse_workspace_bytes(layer, B, 1, Hq, cfg.mode, S, max_tl), dtype=torch.uint8,
                       device=dev)
    E = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731
    rec = {"verify_us": [], "select_us": [], "draft_us": [], "iter_us": [], "recall": [], "moved_rows": []}
    k_flat = k_dev.view(-1, d)
    last = None
    for it in range(-warmup, iters):
        tag = max(it, 0)
        qv = _bf16(torch, synth.make_queries(cfg, kv, cfg.n_q, seed=seed, tag=1000 + 2 * tag), dev)
        qd = [_bf16(torch, synth.make_queries(cfg, kv, 1, seed=seed, tag=100000 + 16 * tag + j), dev)
              for j in range(cfg.n_draft)]
        torch.cuda.synchronize()
        e = [E() for _ in range(4)]
        e[0].record()
        if scores:
            lcs.verify_attn_scores(layer, qv, pl, L, scale, cfg.collect_rows, out=out, scores=logits,
                                   workspace=ws_v)
        else:
            lcs.verify_attn(layer, qv, pl, L, scale, cfg.collect_rows, out=out, logits=logits, workspace=ws_v)
        e[1].record()
        if scores:
            lcs.select_topk_scores(logits, pl, L, cfg.mode, cfg.top_k, cfg.n_sink, cfg.n_recent, cap=S,
                                   indices=idx, counts=cnt, workspace=ws_s, Hq=Hq)
        else:
            lcs.select_topk(logits, pl, L, cfg.Hkv, cfg.mode, cfg.top_k, cfg.n_sink, cfg.n_recent, cap=S,
                            indices=idx, counts=cnt, workspace=ws_s)
        e[2].record()
        for j in range(cfg.n_draft):
            lcs.sparse_draft_attn(layer, qd[j], cfg.mode, idx, cnt, pl, tls[j], max_tl, scale, out=dout,
                                  workspace=ws_d)
        e[3].record()
        torch.cuda.synchronize()
        if it < 0:
            continue
        if keep_last and it == iters - 1:
            last = {"k_before": kv.k.copy(), "q": qv.view(torch.int16).cpu().numpy().view(np.uint16),
                    "qd": qd[-1].view(torch.int16).cpu().numpy().view(np.uint16),
                    "out": out.cpu().numpy(), "logits": logits[..., :L].cpu().numpy(), "idx": idx.cpu().numpy(),
                    "cnt": cnt.cpu().numpy(), "dout": dout.cpu().numpy(),
                    "tail_len": cfg.n_q + cfg.n_draft}
        tv, ts, td = (e[0].elapsed_time(e[1]) * 1e3, e[1].elapsed_time(e[2]) * 1e3,
                      e[2].elapsed_time(e[3]) * 1e3)
        rec["verify_us"].append(tv)
        rec["select_us"].append(ts)
        rec["draft_us"].append(td / max(cfg.n_draft, 1))
        rec["iter_us"].append(tv + ts + td)
        rec["recall"].append(recall(cfg, kv, idx.cpu().numpy(), cnt.cpu().numpy()))
        # drift: move part of every critical set and rewrite the affected K rows
        new_sets = synth.drift_critical(cfg, kv, drift, seed=seed, it=it)
        rows, bits = synth.rewrite_keys(cfg, kv, new_sets, seed=seed, it=it)
        if rows.size:
            k_flat[torch.from_numpy(rows).to(dev)] = _bf16(torch, bits, dev)
        rec["moved_rows"].append(int(rows.size))
        if last is not None:
            torch.cuda.synchronize()
            last["k_after_dev"] = k_dev.view(torch.int16).cpu().numpy().view(np.uint16)
            last["k_after_host"] = kv.k
            last["kv"] = kv
        if log is not None and (it % 32 == 0 or it == iters - 1):
            print(f"iteration {it}: verify {tv:.1f} us, select {ts:.1f} us, draft step {td / max(cfg.n_draft, 1):.1f}"
                  f" us, recall {rec['recall'][-1]:.3f}", file=log, flush=True)
    med = {k: float(np.median(v)) for k, v in rec.items() if v}
    extra = {"last": last} if keep_last else {}
    return {**extra, "config": cfg.name, "iters": iters, "drift": drift, "scores": scores, "median": med,
            "recall_first": rec["recall"][0] if rec["recall"] else None,
            "recall_last": rec["recall"][-1] if rec["recall"] else None,
            "gamma_attn": med["draft_us"] / med["verify_us"] if rec["verify_us"] else None}


def main(argv=None) -> None:
    p = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    p.add_argument("--config", default="stress_128k")
    p.add_argument("--iters", type=int, default=256)
    p.add_argument("--drift", type=float, default=0.1)
    p.add_argument("--seed", type=int, default=0)
    p.add_argument("--scores", action="store_true", help="per-KV-head partial scores instead of logit rows")
    a = p.parse_args(argv)
    from . import synth
    t0 = time.time()
    res = run(synth.CONFIGS[a.config], a.iters, a.drift, a.seed, log=sys.stderr, scores=a.scores)
    res["wall_s"] = round(time.time() - t0, 1)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
