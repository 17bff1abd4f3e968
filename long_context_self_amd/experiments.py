"""Measurements of the scoring variants on synthetic workloads.

    python -m long_context_self_amd.experiments collect-overhead --config llama8b_32k
    python -m long_context_self_amd.experiments overlap --config llama8b_32k
    python -m long_context_self_amd.experiments row-scaling --config llama8b_32k
    python -m long_context_self_amd.experiments block-merge --config nsa_16k
    python -m long_context_self_amd.experiments latency --config llama8b_32k
    python -m long_context_self_amd.experiments layer-stack [--layers 16] [--context 32768]

collect-overhead: verify latency against the number of collected logit rows (none,
one, the two boundary rows, half, all n_q).  The Vegas page (Figure 6 and its text)
reports that collecting more rows slows verification through memory-bandwidth
contention and keeps two for that reason; this is the same curve for these kernels.
Each call runs on a KV replica last touched several calls earlier, so it reads HBM.

overlap: how far the selected sets of the scoring variants agree, and how many of
the planted critical positions each one holds.  The Vegas page (Figure 7, Table 1)
compares the boundary-row selection with one driven by every verifier row; the
Sparse Glimpse page scores by the post-softmax weights of the last verification
queries.  Overlap counts the top-k part only (the sink and recent windows are the
same for every variant) against the all-row logit selection.

row-scaling: verify latency against the number of verifier rows, up to 64 (trees of
many drafts, SSV page), on the workload's shapes.

block-merge: SSV block mode (section 4.2 of the SSV page): the tree's rows in one call,
which loads the union of their block sets once, against each row alone.

nsa: NSA sparse verification (SSV page, Figure 3 and Figure 10): compression, the
block plan, and the fused three-branch attention with exact, approximate or no
grouping of the tree's rows.

latency: p10 / p50 / p90 of every call over 100 calls, each after a 512 MiB cache
flush, with GB/s against the 8 TB/s peak and against a measured device copy.

layer-stack: forward latency of a random-weight Llama-3.2-1B-shaped stack at 32K
context against the draft length, with dense verification or NSA sparse
verification as its attention (SSV page, Figure 7; `layer_stack`).

Host orchestration only: every step runs in the library's kernels.  Inputs are the
seeded synthetic workloads of `synth`; the numbers are properties of those inputs,
not of any dataset.
"""
from __future__ import annotations

import argparse
import json
import math
import sys

import numpy as np


def _dev_inputs(torch, cfg, seed, replicas):
    from . import lcs, synth
    kv = synth.make_paged_kv(cfg, seed=seed)
    q = synth.make_queries(cfg, kv, cfg.n_q, seed=seed)

    def bf16(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to("cuda")

    k0, v0 = bf16(kv.k), bf16(kv.v)
    bt = torch.from_numpy(kv.block_table).to("cuda")
    layers = [lcs.PagedKV(k0 if r == 0 else k0.clone(), v0 if r == 0 else v0.clone(), bt) for r in range(replicas)]
    return kv, layers, bf16(q), torch.from_numpy(kv.prefix_len).to("cuda")


def collect_overhead(cfg, replicas: int, iters: int, seed: int = 0) -> dict:
    import torch

    from . import lcs
    kv, layers, q, pl = _dev_inputs(torch, cfg, seed, replicas)
    B, Hq, L, n_q = cfg.B, cfg.Hq, cfg.L, cfg.n_q
    scale = 1.0 / math.sqrt(cfg.d)
    sets = {"0": [], "1": [n_q - 1], "2": [0, n_q - 1], "half": list(range(0, n_q, 2)), "all": list(range(n_q))}
    out = torch.empty((B, n_q, Hq, cfg.d), dtype=torch.float32, device="cuda")
    lse = torch.empty((B, n_q, Hq), dtype=torch.float32, device="cuda")
    ws = torch.empty(lcs.verify_workspace_bytes(layers[0], B, n_q, Hq, L), dtype=torch.uint8, device="cuda")
    res = {}
    for name, rows in sets.items():
        lg = (torch.empty((B, Hq, len(rows), lcs.row_ld(L)), dtype=torch.float32, device="cuda") if rows else None)

        def call(r):
            lcs.verify_attn_rows(layers[r], q, pl, L, scale, rows or [0], out=out, logits=lg, lse=lse,
                                 workspace=ws, with_logits=bool(rows))
        for r in range(replicas):
            call(r)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(iters):
            for r in range(replicas):
                call(r)
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / (iters * replicas)
        kv_bytes = 4 * B * cfg.Hkv * cfg.d * (L + n_q)
        res[name] = {"rows": len(rows), "verify_us": round(us, 2),
                     "logit_bytes_over_kv": round(4 * B * Hq * len(rows) * L / kv_bytes, 4)}
        del lg
    base = res["0"]["verify_us"]
    for v in res.values():
        v["overhead"] = round(v["verify_us"] / base - 1.0, 4)
    return {"config": cfg.name, "replicas": replicas, "iters": iters, "points": res}


def row_scaling(cfg, replicas: int, iters: int, n_qs=(9, 16, 17, 33, 64), seed: int = 0) -> dict:
    """Verify latency against the number of verifier rows (trees of up to 64 drafts),
    the two boundary rows collected, on the workload's shapes with n_q replaced."""
    import torch

    from . import lcs
    res = {}
    for n_q in n_qs:
        c = cfg.with_(n_q=n_q, n_draft=n_q - 1)
        kv, layers, q, pl = _dev_inputs(torch, c, seed, replicas)
        B, Hq, L = c.B, c.Hq, c.L
        scale = 1.0 / math.sqrt(c.d)
        out = torch.empty((B, n_q, Hq, c.d), dtype=torch.float32, device="cuda")
        lg = torch.empty((B, Hq, 2, lcs.row_ld(L)), dtype=torch.float32, device="cuda")
        ws = torch.empty(lcs.verify_workspace_bytes(layers[0], B, n_q, Hq, L), dtype=torch.uint8, device="cuda")

        def call(r):
            lcs.verify_attn(layers[r], q, pl, L, scale, (0, n_q - 1), out=out, logits=lg, workspace=ws)
        for r in range(replicas):
            call(r)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(iters):
            for r in range(replicas):
                call(r)
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / (iters * replicas)
        res[str(n_q)] = {"rows_per_kv_group": n_q * c.G, "verify_us": round(us, 2)}
        del layers, kv, lg, out, ws
        torch.cuda.empty_cache()
    return {"config": cfg.name, "replicas": replicas, "iters": iters, "points": res}


def block_merge(cfg, replicas: int, iters: int, seed: int = 0) -> dict:
    """SSV block mode: the n_q tree rows in one call (the union of their block sets loaded
    once) against each row alone (n_q calls, every row's blocks loaded for it)."""
    import torch

    from . import lcs, synth
    kv = synth.make_paged_kv(cfg, seed=seed)
    nblk = cfg.L // cfg.page_size
    sets = synth.make_block_sets(cfg, nblk, seed=seed)
    q_np = synth.make_queries(cfg, kv, cfg.n_q, seed=seed)
    tm_np = np.stack([synth.tree_tail_masks(cfg.n_q, cfg.tree_branches)] * cfg.B)

    def bf16(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to("cuda")

    k0, v0 = bf16(kv.k), bf16(kv.v)
    bt = torch.from_numpy(kv.block_table).to("cuda")
    layers = [lcs.PagedKV(k0 if r == 0 else k0.clone(), v0 if r == 0 else v0.clone(), bt) for r in range(replicas)]
    B, n_q, Hq, d = cfg.B, cfg.n_q, cfg.Hq, cfg.d
    q = bf16(q_np)
    idx = torch.from_numpy(sets).to("cuda")
    cnt = torch.full((B, n_q, cfg.Hkv), cfg.blocks_per_row, dtype=torch.int32, device="cuda")
    tb = torch.from_numpy(kv.prefix_len).to("cuda")
    tl = torch.full((B,), n_q, dtype=torch.int32, device="cuda")
    tm = torch.from_numpy(tm_np.view(np.int64)).to("cuda")
    scale = 1.0 / math.sqrt(d)
    rows = [(q[:, i:i + 1].contiguous(), idx[:, i:i + 1].contiguous(), cnt[:, i:i + 1].contiguous(),
             tm[:, i:i + 1].contiguous()) for i in range(n_q)]
    out = torch.empty((B, n_q, Hq, d), dtype=torch.float32, device="cuda")
    out1 = torch.empty((B, 1, Hq, d), dtype=torch.float32, device="cuda")

    def merged(r):
        lcs.sparse_draft_attn(layers[r], q, "block", idx, cnt, tb, tl, n_q, scale, tail_mask=tm, out=out)

    def unmerged(r):
        for qi, ii, ci, ti in rows:
            lcs.sparse_draft_attn(layers[r], qi, "block", ii, ci, tb, tl, n_q, scale, tail_mask=ti, out=out1)

    res = {}
    for name, fn in (("merged", merged), ("unmerged", unmerged)):
        for r in range(replicas):
            fn(r)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(iters):
            for r in range(replicas):
                fn(r)
        e1.record()
        torch.cuda.synchronize()
        res[name] = {"us": round(e0.elapsed_time(e1) * 1e3 / (iters * replicas), 2)}
    # algorithmic K/V bytes: the union of the rows' blocks per (b, g) when merged, every
    # row's own blocks when not (the tail of n_q tokens is read in both)
    P = cfg.page_size
    union = sum(len(np.unique(sets[b, :, g])) for b in range(B) for g in range(cfg.Hkv))
    per_row = int(B * cfg.Hkv * n_q * cfg.blocks_per_row)
    tail = B * cfg.Hkv * n_q
    res["merged"]["kv_bytes"] = 4 * d * (P * union + tail)
    res["unmerged"]["kv_bytes"] = 4 * d * (P * per_row + n_q * tail)
    for v in res.values():
        v["GB/s"] = round(v["kv_bytes"] / (v["us"] * 1e3), 1)
    res["mean_union_blocks"] = round(union / (B * cfg.Hkv), 2)
    return {"config": cfg.name, "replicas": replicas, "iters": iters, "points": res}


def nsa(cfg, replicas: int, iters: int, seed: int = 0) -> dict:
    """NSA sparse verification on the SSV workload: the compression pass, the block plan
    (index derivation of a refresh layer), and the fused three-branch attention with the
    rows grouped exactly, approximately, or not at all (each row alone, with its own plan),
    each call on a KV replica last touched several calls earlier."""
    import torch

    from . import lcs, synth
    from .metrics import nsa_bytes
    kv = synth.make_paged_kv(cfg, seed=seed, extra_tokens=cfg.n_q)
    nblk = cfg.L // cfg.page_size
    sets = synth.make_block_sets(cfg, nblk, seed=seed)
    q_np = synth.make_queries(cfg, kv, cfg.n_q, seed=seed)
    tm_np = np.stack([synth.tree_tail_masks(cfg.n_q, cfg.tree_branches)] * cfg.B)
    gates_np = synth.make_gates(cfg, cfg.n_q, seed=seed)

    def bf16(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to("cuda")

    k0, v0 = bf16(kv.k), bf16(kv.v)
    bt = torch.from_numpy(kv.block_table).to("cuda")
    layers = [lcs.PagedKV(k0 if r == 0 else k0.clone(), v0 if r == 0 else v0.clone(), bt) for r in range(replicas)]
    B, n_q, Hq, d = cfg.B, cfg.n_q, cfg.Hq, cfg.d
    pl = torch.from_numpy(kv.prefix_len).to("cuda")
    max_cmp = (cfg.L - cfg.cmp_len) // cfg.cmp_stride + 1
    comp = [lcs.nsa_compress(layers[r], pl, cfg.L, cfg.cmp_len, cfg.cmp_stride, max_cmp) for r in range(replicas)]
    q = bf16(q_np)
    idx = torch.from_numpy(sets).to("cuda")
    cnt = torch.full((B, n_q, cfg.Hkv), cfg.blocks_per_row, dtype=torch.int32, device="cuda")
    tl = torch.full((B,), n_q, dtype=torch.int32, device="cuda")
    tm = torch.from_numpy(tm_np.view(np.int64)).to("cuda")
    gates = torch.from_numpy(gates_np).to("cuda")
    scale = 1.0 / math.sqrt(d)
    plans = {grp: lcs.nsa_plan(layers[0], idx, cnt, grp) for grp in ("exact", "approximate")}
    rows = []
    for i in range(n_q):
        ii, ci = idx[:, i:i + 1].contiguous(), cnt[:, i:i + 1].contiguous()
        rows.append((q[:, i:i + 1].contiguous(), ii, ci, lcs.nsa_plan(layers[0], ii, ci),
                     gates[:, i:i + 1].contiguous(), tm[:, i:i + 1].contiguous()))
    out = torch.empty((B, n_q, Hq, d), dtype=torch.float32, device="cuda")
    out1 = torch.empty((B, 1, Hq, d), dtype=torch.float32, device="cuda")
    ws = torch.empty(lcs.nsa_workspace_bytes(layers[0], B, n_q, Hq, cfg.blocks_per_row, n_q, max_cmp, cfg.window),
                     dtype=torch.uint8, device="cuda")

    def attn(r, grp):
        lcs.nsa_attn(layers[r], comp[r][0], comp[r][1], cfg.cmp_len, cfg.cmp_stride, cfg.window, q, plans[grp],
                     cfg.blocks_per_row, pl, tl, n_q, gates, scale, tail_mask=tm, out=out, workspace=ws)

    def per_row(r):
        for qi, ii, ci, pi, gi, ti in rows:
            lcs.nsa_plan(layers[r], ii, ci, plan=pi)
            lcs.nsa_attn(layers[r], comp[r][0], comp[r][1], cfg.cmp_len, cfg.cmp_stride, cfg.window, qi, pi,
                         cfg.blocks_per_row, pl, tl, n_q, gi, scale, tail_mask=ti, out=out1, workspace=ws)

    calls = {
        "compress": lambda r: lcs.nsa_compress(layers[r], pl, cfg.L, cfg.cmp_len, cfg.cmp_stride, max_cmp,
                                               k_cmp=comp[r][0], v_cmp=comp[r][1]),
        "plan (refresh layer)": lambda r: lcs.nsa_plan(layers[r], idx, cnt, plan=plans["exact"]),
        "attention, exact grouping (reuse layer)": lambda r: attn(r, "exact"),
        "attention, approximate grouping": lambda r: attn(r, "approximate"),
        "no grouping (each row: plan + attention)": per_row,
    }
    res = {}
    for name, fn in calls.items():
        for r in range(replicas):
            fn(r)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(iters):
            for r in range(replicas):
                fn(r)
        e1.record()
        torch.cuda.synchronize()
        res[name] = {"us": round(e0.elapsed_time(e1) * 1e3 / (iters * replicas), 2)}
    union = sum(len(np.unique(sets[b, :, g])) for b in range(B) for g in range(cfg.Hkv))
    by = nsa_bytes(cfg, union, max_cmp)
    for name in ("attention, exact grouping (reuse layer)", "attention, approximate grouping"):
        res[name]["bytes"] = by
        res[name]["GB/s"] = round(by / (res[name]["us"] * 1e3), 1)
    return {"config": cfg.name, "replicas": replicas, "iters": iters, "max_cmp": max_cmp,
            "mean_union_blocks": round(union / (B * cfg.Hkv), 2), "points": res}


def latency(cfg, calls: int = 100, warmup: int = 10, flush_mib: int = 512, seed: int = 0,
            flush: str = "read") -> dict:
    """p10 / p50 / p90 latency of each call under a cold-cache protocol: before every
    timed call a 512 MiB scratch buffer passes through the caches (outside the timed
    events), which evicts the 256 MB Infinity Cache and the L2s.  flush "read" reads a
    clean buffer; "write" writes it, which leaves the caches full of dirty lines that
    the timed call then pays to write back.  GB/s is the call's algorithmic bytes over
    its p50, against the 8 TB/s peak and against a measured device copy."""
    import torch

    from . import lcs, metrics, synth
    kv, layers, q, pl = _dev_inputs(torch, cfg, seed, 1)
    layer = layers[0]

    def bf16(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to("cuda")

    qd = bf16(synth.make_queries(cfg, kv, 1, seed=seed, tag=100))
    B, Hq, L, d = cfg.B, cfg.Hq, cfg.L, cfg.d
    scale = 1.0 / math.sqrt(d)
    n_sets = 1 if cfg.mode == "shared" else cfg.Hkv
    S = cfg.n_sink + cfg.top_k + cfg.n_recent
    tail = cfg.n_q + 1
    out = torch.empty((B, cfg.n_q, Hq, d), dtype=torch.float32, device="cuda")
    lse = torch.empty((B, cfg.n_q, Hq), dtype=torch.float32, device="cuda")
    lg = torch.empty((B, Hq, 2, lcs.row_ld(L)), dtype=torch.float32, device="cuda")
    idx = torch.empty((B, n_sets, S), dtype=torch.int32, device="cuda")
    cnt = torch.empty((B, n_sets), dtype=torch.int32, device="cuda")
    dout = torch.empty((B, 1, Hq, d), dtype=torch.float32, device="cuda")
    tl = torch.full((B,), tail, dtype=torch.int32, device="cuda")
    ws_v = torch.empty(lcs.verify_workspace_bytes(layer, B, cfg.n_q, Hq, L), dtype=torch.uint8, device="cuda")
    ws_s = torch.empty(lcs.select_workspace_bytes(B, Hq, cfg.Hkv, cfg.mode, L), dtype=torch.uint8, device="cuda")
    ws_d = torch.empty(lcs.sparse_workspace_bytes(layer, B, 1, Hq, cfg.mode, S, tail), dtype=torch.uint8,
                       device="cuda")
    calls_fn = {
        "verify": lambda: lcs.verify_attn(layer, q, pl, L, scale, cfg.collect_rows, out=out, logits=lg, lse=lse,
                                          workspace=ws_v),
        "select": lambda: lcs.select_topk(lg, pl, L, cfg.Hkv, cfg.mode, cfg.top_k, cfg.n_sink, cfg.n_recent, cap=S,
                                          indices=idx, counts=cnt, workspace=ws_s),
        "draft_step": lambda: lcs.sparse_draft_attn(layer, qd, cfg.mode, idx, cnt, pl, tl, tail, scale, out=dout,
                                                    workspace=ws_d),
    }
    scratch = torch.ones(flush_mib << 17, dtype=torch.int64, device="cuda")
    sink = torch.empty((), dtype=torch.int64, device="cuda")

    def do_flush(c):
        if flush == "write":
            scratch.fill_(c)
        else:
            torch.sum(scratch, dim=0, out=sink)
    for c in range(3):          # the buffer's own first writes leave the caches first
        do_flush(c)
    # measured streaming bandwidth: a device copy of 1 GiB (read + write)
    src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(5):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    copy_gbs = 5 * 2 * src.numel() / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del src, dst
    res = {}
    for name, fn in calls_fn.items():
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        ev = []
        for c in range(calls):
            do_flush(c)
            a, z = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            fn()
            z.record()
            ev.append((a, z))
        torch.cuda.synchronize()
        us = np.array([a.elapsed_time(z) * 1e3 for a, z in ev])
        p10, p50, p90 = (float(np.percentile(us, x)) for x in (10, 50, 90))
        nbytes = {"verify": metrics.verify_bytes(cfg), "select": metrics.select_bytes(cfg, S),
                  "draft_step": metrics.draft_bytes(cfg, S, tail)}[name]
        gbs = nbytes / (p50 * 1e3)
        res[name] = {"p10_us": round(p10, 2), "p50_us": round(p50, 2), "p90_us": round(p90, 2), "bytes": nbytes,
                     "GB/s_p50": round(gbs, 1), "frac_8TBps": round(gbs / metrics.HBM_PEAK_GBS, 4),
                     "frac_copy": round(gbs / copy_gbs, 4)}
    return {"config": cfg.name, "calls": calls, "warmup": warmup, "flush_MiB": flush_mib, "flush": flush,
            "copy_GBps": round(copy_gbs, 1), "calls_us": res}


def _topk_part(idx, cnt, b, s, L, cfg):
    sel = idx[b, s, :int(cnt[b, s])]
    return sel[(sel >= cfg.n_sink) & (sel < L - cfg.n_recent)]


def overlap(cfg, seed: int = 0) -> dict:
    import torch

    from . import lcs
    kv, layers, q, pl = _dev_inputs(torch, cfg, seed, 1)
    n_q, L = cfg.n_q, cfg.L
    scale = 1.0 / math.sqrt(cfg.d)
    W = min(16, n_q)
    rows_all = list(range(n_q))
    _, lg_all, lse = lcs.verify_attn_rows(layers[0], q, pl, L, scale, rows_all)
    variants = {
        "all_rows_logits": (rows_all, "logits"),
        "boundary_rows_logits": ([0, n_q - 1], "logits"),
        "first_row_logits": ([0], "logits"),
        "last_row_logits": ([n_q - 1], "logits"),
        "last_W_rows_weights": (list(range(n_q - W, n_q)), "weights"),
        "boundary_rows_weights": ([0, n_q - 1], "weights"),
    }
    sel = {}
    for name, (rows, kind) in variants.items():
        lg = lg_all[:, :, rows].contiguous()
        idx, cnt = lcs.select_topk_rows(lg, pl, L, cfg.Hkv, cfg.mode, cfg.top_k, cfg.n_sink, cfg.n_recent,
                                        score=kind, lse=lse, rows=rows)
        torch.cuda.synchronize()
        sel[name] = (idx.cpu().numpy(), cnt.cpu().numpy())
    n_sets = 1 if cfg.mode == "shared" else cfg.Hkv
    ref_i, ref_c = sel["all_rows_logits"]
    res = {}
    for name, (idx, cnt) in sel.items():
        ov, rec = [], []
        for b in range(cfg.B):
            Lb = int(kv.prefix_len[b])
            for s in range(n_sets):
                a = _topk_part(idx, cnt, b, s, Lb, cfg)
                r = _topk_part(ref_i, ref_c, b, s, Lb, cfg)
                if r.size:
                    ov.append(np.isin(a, r).sum() / r.size)
            for g in range(cfg.Hkv):
                crit = kv.critical[b][g]
                if crit.size:
                    s = 0 if cfg.mode == "shared" else g
                    rec.append(np.isin(crit, idx[b, s, :int(cnt[b, s])]).mean())
        res[name] = {"rows": variants[name][0], "score": variants[name][1],
                     "overlap_with_all_rows": round(float(np.mean(ov)), 4),
                     "critical_recall": round(float(np.mean(rec)), 4) if rec else None}
    blind = (cfg.n_sink + cfg.top_k + cfg.n_recent) / cfg.L
    return {"config": cfg.name, "mode": cfg.mode, "top_k": cfg.top_k, "blind_recall": round(blind, 4),
            "variants": res}


def main(argv=None) -> None:
    p = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    p.add_argument("what", choices=["collect-overhead", "overlap", "row-scaling", "block-merge", "latency",
                                    "layer-stack", "nsa"])
    p.add_argument("--layers", type=int, default=16, help="layer-stack: layers")
    p.add_argument("--context", type=int, default=32768, help="layer-stack: prefix length")
    p.add_argument("--config", default="llama8b_32k")
    p.add_argument("--replicas", type=int, default=0, help="KV copies rotated per timed call (0: sized to ~2 GB)")
    p.add_argument("--iters", type=int, default=5)
    p.add_argument("--seed", type=int, default=0)
    p.add_argument("--flush", choices=["read", "write"], default="read", help="latency: how the caches are flushed")
    a = p.parse_args(argv)
    if a.what == "layer-stack":
        from . import layer_stack
        shape = layer_stack.StackShape(layers=a.layers, context=a.context)
        print(json.dumps(layer_stack.run(shape, iters=a.iters, seed=a.seed, log=sys.stderr)), flush=True)
        return
    from . import synth
    cfg = synth.CONFIGS[a.config]
    kv_bytes = 4 * cfg.B * cfg.Hkv * cfg.d * cfg.L
    reps = a.replicas or max(2, min(16, int(2e9 // kv_bytes)))
    if a.what == "collect-overhead":
        res = collect_overhead(cfg, reps, a.iters, a.seed)
    elif a.what == "row-scaling":
        res = row_scaling(cfg, reps, a.iters, seed=a.seed)
    elif a.what == "block-merge":
        res = block_merge(cfg, reps, a.iters, seed=a.seed)
    elif a.what == "latency":
        res = latency(cfg, seed=a.seed, flush=a.flush)
    elif a.what == "nsa":
        res = nsa(cfg, reps, a.iters, seed=a.seed)
    else:
        res = overlap(cfg, a.seed)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    sys.exit(main())
