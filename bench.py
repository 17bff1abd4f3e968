"""Benchmark of the verify / select / sparse-draft attention path on one MI355X.

One step is one speculative decode iteration of the attention hot path of an
n-layer model.  The default workload is the largest one-GPU configuration, the
long-context stress shape (8 sequences of 131072 tokens, 32 query / 8 KV heads,
head dim 128, draft length 8, shared top-4096 + 4 sink + 64 recent), over 4 layers:

    for each of the k draft steps:  sparse_draft_attn on every layer
    for every layer:                verify_attn (k+1 rows, two logit rows collected)
    for every layer:                select_topk (next iteration's sparse set)

Every layer owns its own KV cache copy, so consecutive calls on one layer are
separated by the other layers' traffic (several GB) and read HBM, not the
256 MB Infinity Cache; this is the situation of a real multi-layer model.

Prints one JSON line.  `value` is the achieved algorithmic HBM bandwidth of the
whole step (bytes the method must move / step time); the per-call latencies in
microseconds and their fractions of the 8 TB/s peak are in `kernels`.  `roofline`
is for the call with the largest share of the step's time.  `secondary` repeats the
per-call measurement on the Llama-3-8B-shaped layer at 32K context (32 layers).
`cpu_baseline` times the fp64 oracle on a bounded sample of the main workload.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0   # the peak line every fraction is taken against (metrics.HBM_PEAK_GBS)
DEFAULT_CONFIG = "stress_128k"
DEFAULT_LAYERS = {"stress_128k": 4, "qwen14b_64k": 4, "llama8b_32k": 32, "tiny": 4}
SECONDARY_CONFIG = "llama8b_32k"


def traffic_file(workload: str, call: str) -> str:
    """Committed counter-traffic summary of one call on one workload (rocprofv3 runs)."""
    return os.path.join(ROOT, "profiles", f"{call}_{workload}_traffic.json")


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--config", default=DEFAULT_CONFIG)
    p.add_argument("--layers", type=int, default=0,
                   help="layers (KV replicas); 0 = the workload's default (4 at 128K x 8, 32 at 32K)")
    p.add_argument("--no-variants", action="store_true",
                   help="skip the fused variants (partial scores, physical hand-off) on the same inputs")
    p.add_argument("--no-secondary", action="store_true",
                   help="skip the secondary per-call measurement on the 32K workload")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=15.0)
    p.add_argument("--refresh-every", type=int, default=1,
                   help="SSV refresh/reuse schedule: select on every R-th layer only; the layers between "
                        "reuse the nearest preceding refresh layer's sets")
    p.add_argument("--oracle-timing", action="store_true",
                   help="only time the fp64 oracle per call on every workload (host cores, no GPU)")
    p.add_argument("--scores", action="store_true",
                   help="verify writes per-KV-head partial scores and select reads them, instead of the "
                        "two collected logit rows")
    p.add_argument("--physical", action="store_true",
                   help="select hands its sets to the draft as physical cache slots (the fused hand-off)")
    p.add_argument("--copy-calibration-mib", type=int, default=0,
                   help="run one device-to-device copy of this size first (counter calibration)")
    return p.parse_args()


def algorithmic_bytes(cfg, S_draft, tail_lens, scores=False):
    """Bytes each call must move at minimum (long_context_self_amd.metrics)."""
    from long_context_self_amd import metrics
    return (metrics.verify_bytes(cfg, scores), metrics.select_bytes(cfg, S_draft, scores),
            [metrics.draft_bytes(cfg, S_draft, tl) for tl in tail_lens])


def traffic_record(workload: str, call: str):
    """HBM bytes per call from committed rocprofv3 counter runs of this workload, if
    they were taken on the current kernel source (else None)."""
    try:
        rec = json.load(open(traffic_file(workload, call)))
    except (OSError, ValueError):
        return None
    from long_context_self_amd.profile_summary import kernel_source_hash
    if rec.get("kernel_source_hash") != kernel_source_hash():
        return None
    return rec.get("hbm_bytes_per_launch")


def cpu_baseline(cfg, budget_s):
    """fp64 oracle on a bounded sample of the workload: rounds of one sequence and one KV
    head of one layer (verify for its G query heads, the set's select, and the k draft
    steps), on inputs drawn like the workload's.  The select leg needs every query head's
    two rows for a shared set; the sample has G heads, so their rows stand in for the
    other groups' (replicated), which costs the same work as the real rows."""
    from long_context_self_amd import synth
    from oracle import attention as oa
    from oracle import select as osel
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = os.cpu_count() or 1
    one = cfg.with_(B=1, Hkv=1, Hq=cfg.G)            # one sequence, one KV group
    kv = synth.make_paged_kv(one, seed=0)
    q = synth.make_queries(one, kv, one.n_q, seed=0)
    qd = [synth.make_queries(one, kv, 1, seed=0, tag=100 + j) for j in range(one.n_draft)]
    scale = 1.0 / math.sqrt(cfg.d)
    n_sets = 1 if cfg.mode == "shared" else cfg.Hkv
    heads = cfg.Hq if cfg.mode == "shared" else cfg.G
    bytes_done = 0
    rounds = 0
    t0 = time.perf_counter()
    while True:
        _, lg, _ = oa.verify_attn(q, kv.k, kv.v, kv.block_table, kv.prefix_len, one.page_size, scale)
        full_lg = np.repeat(lg, heads // cfg.G, axis=1)   # stand-in rows for the set's other heads
        sel = osel.select(full_lg, kv.prefix_len, 1, "shared", cfg.top_k, cfg.n_sink, cfg.n_recent)
        i_, c_ = osel.pack(sel, max(a.size for r in sel for a in r))
        for j in range(cfg.n_draft):
            tl = np.full(1, cfg.n_q + j + 1, dtype=np.int32)
            oa.sparse_attn(qd[j], kv.k, kv.v, kv.block_table, one.page_size, "shared", i_, c_,
                           kv.prefix_len, tl, scale)
        S = int(c_[0, 0])
        v_b, s_b, d_b = algorithmic_bytes(cfg, S, [cfg.n_q + j + 1 for j in range(cfg.n_draft)])
        pairs = cfg.B * cfg.Hkv
        bytes_done += (v_b + sum(d_b)) / pairs + s_b / (cfg.B * n_sets)
        rounds += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    return {"value": round(bytes_done / dt / 1e9, 4), "unit": "GB/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"{rounds} rounds of one sequence x one KV head (G={cfg.G} query heads) of one "
                      f"{cfg.name} layer: verify, the set's select (the G heads' logit rows replicated to "
                      f"stand in for the set's {heads} heads), {cfg.n_draft} draft steps; fp64 NumPy, "
                      f"{dt:.1f} s; bytes counted as that share of the workload's algorithmic bytes"}


def oracle_timing():
    """The fp64 oracle timed per call on every workload (host cores only, no GPU): one
    (sequence, KV head) sample of each call, scaled to the whole call."""
    from long_context_self_amd import synth
    from oracle import attention as oa
    from oracle import select as osel
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = os.cpu_count() or 1
    res = {}
    for name in ("tiny", "llama8b_32k", "qwen14b_64k", "nsa_16k", "stress_128k"):
        cfg = synth.CONFIGS[name].with_(B=1)            # one sequence of the workload
        full = synth.CONFIGS[name]
        kv = synth.make_paged_kv(cfg, seed=0)
        q = synth.make_queries(cfg, kv, cfg.n_q, seed=0)[:, :, :cfg.G]
        k1, v1 = kv.k[:, :1], kv.v[:, :1]                # one KV head
        scale = 1.0 / math.sqrt(cfg.d)
        pairs = full.B * full.Hkv
        rec = {}
        if cfg.mode == "block":
            nblk = cfg.L // cfg.page_size
            sets = synth.make_block_sets(cfg, nblk, seed=0)[:, :, :1]
            cnt = np.full((1, cfg.n_q, 1), cfg.blocks_per_row, dtype=np.int32)
            tm = synth.tree_tail_masks(cfg.n_q, cfg.tree_branches)[None]
            t0 = time.perf_counter()
            oa.sparse_attn(q, k1, v1, kv.block_table, cfg.page_size, "block", sets, cnt, kv.prefix_len,
                           np.full(1, cfg.n_q, np.int32), scale, tail_mask=tm)
            rec["block_sparse_s"] = round((time.perf_counter() - t0) * pairs, 4)
        else:
            t0 = time.perf_counter()
            _, lg, _ = oa.verify_attn(q, k1, v1, kv.block_table, kv.prefix_len, cfg.page_size, scale)
            rec["verify_s"] = round((time.perf_counter() - t0) * pairs, 4)
            heads = full.Hq if full.mode == "shared" else cfg.G
            lg_full = np.repeat(lg, heads // cfg.G, axis=1)  # stand-in rows for the set's other heads
            t0 = time.perf_counter()
            sel = osel.select(lg_full, kv.prefix_len, 1, "shared", cfg.top_k, cfg.n_sink, cfg.n_recent)
            n_sets = 1 if full.mode == "shared" else full.Hkv
            rec["select_s"] = round((time.perf_counter() - t0) * full.B * n_sets, 4)
            i_, c_ = osel.pack(sel, max(a.size for r in sel for a in r))
            qd = synth.make_queries(cfg, kv, 1, seed=0, tag=100)[:, :, :cfg.G]
            t0 = time.perf_counter()
            oa.sparse_attn(qd, k1, v1, kv.block_table, cfg.page_size, "shared", i_, c_, kv.prefix_len,
                           np.full(1, cfg.n_q + 1, np.int32), scale)
            rec["draft_step_s"] = round((time.perf_counter() - t0) * pairs, 4)
            rec["iteration_s"] = round(rec["verify_s"] + rec["select_s"] + full.n_draft * rec["draft_step_s"], 4)
        n_sets_all = full.B * (1 if full.mode == "shared" else full.Hkv)
        rec["sample"] = (f"one sequence x one KV head of {name}: attention scaled x{pairs} (sequences x KV "
                         f"heads), select x{n_sets_all} (sequences x sets)")
        res[name] = rec
        print(f"{name}: {rec}", file=sys.stderr, flush=True)
        del kv
    print(json.dumps({"oracle_timing": res, "cores": int(threads), "kind": "oracle", "precision": "fp64"}),
          flush=True)


def setup_workload(cfg, R, copy_calibration_mib=0, log=None):
    """Device inputs of workload cfg over R layers (each layer its own KV replica)."""
    import torch

    from long_context_self_amd import lcs, synth

    assert cfg.mode in ("shared", "per_kv_head"), "bench covers the token-set workloads"
    dev = "cuda"
    t_setup = time.perf_counter()
    kv = synth.make_paged_kv(cfg, seed=0)
    q = synth.make_queries(cfg, kv, cfg.n_q, seed=0)
    qd = [synth.make_queries(cfg, kv, 1, seed=0, tag=100 + j) for j in range(cfg.n_draft)]

    def bf16(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)

    k0, v0 = bf16(kv.k), bf16(kv.v)
    bt = torch.from_numpy(kv.block_table).to(dev)
    pl = torch.from_numpy(kv.prefix_len).to(dev)
    del kv
    layers = [lcs.PagedKV(k0 if r == 0 else k0.clone(), v0 if r == 0 else v0.clone(), bt) for r in range(R)]
    if copy_calibration_mib > 0:
        src = torch.empty(copy_calibration_mib << 20, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    torch.cuda.synchronize()
    if log:
        print(f"{cfg.name}: set up {R} layers in {time.perf_counter() - t_setup:.1f} s", file=log, flush=True)
    return {"cfg": cfg, "R": R, "layers": layers, "qv": bf16(q), "qds": [bf16(x) for x in qd], "pl": pl}


def measure(ws, steps, warmup, scores=False, refresh_every=1, physical=False):
    """Time `steps` bench steps on the set-up workload ws.  Returns the per-call latencies
    (us, HIP events on the calling stream), the algorithmic bytes and the step time."""
    import torch

    from long_context_self_amd import lcs

    cfg, R, layers, qv, qds, pl = ws["cfg"], ws["R"], ws["layers"], ws["qv"], ws["qds"], ws["pl"]
    dev = "cuda"
    scale = 1.0 / math.sqrt(cfg.d)
    B, Hq, L = cfg.B, cfg.Hq, cfg.L
    n_sets = 1 if cfg.mode == "shared" else cfg.Hkv
    S = cfg.n_sink + cfg.top_k + cfg.n_recent
    outs = torch.empty((B, cfg.n_q, Hq, cfg.d), dtype=torch.float32, device=dev)
    lses = torch.empty((B, cfg.n_q, Hq), dtype=torch.float32, device=dev)
    if scores:
        logits = [torch.empty((B, cfg.Hkv, lcs.row_ld(L)), dtype=torch.float32, device=dev) for _ in range(R)]
    else:
        logits = [torch.empty((B, Hq, 2, lcs.row_ld(L)), dtype=torch.float32, device=dev) for _ in range(R)]
    idx = [torch.empty((B, n_sets, S), dtype=torch.int32, device=dev) for _ in range(R)]
    cnt = [torch.empty((B, n_sets), dtype=torch.int32, device=dev) for _ in range(R)]
    dout = torch.empty((B, 1, Hq, cfg.d), dtype=torch.float32, device=dev)
    dlse = torch.empty((B, 1, Hq), dtype=torch.float32, device=dev)
    tls = [torch.full((B,), cfg.n_q + j + 1, dtype=torch.int32, device=dev) for j in range(cfg.n_draft)]
    max_tl = cfg.n_q + cfg.n_draft
    ws_v = torch.empty(lcs.verify_workspace_bytes(layers[0], B, cfg.n_q, Hq, L), dtype=torch.uint8, device=dev)
    ws_s = torch.empty(lcs.select_workspace_bytes(B, Hq, cfg.Hkv, cfg.mode, L), dtype=torch.uint8, device=dev)
    ws_d = torch.empty(lcs.sparse_workspace_bytes(layers[0], B, 1, Hq, cfg.mode, S, max_tl),
                       dtype=torch.uint8, device=dev)

    def verify(r):
        if scores:
            lcs.verify_attn_scores(layers[r], qv, pl, L, scale, cfg.collect_rows, out=outs, scores=logits[r],
                                   lse=lses, workspace=ws_v)
        else:
            lcs.verify_attn(layers[r], qv, pl, L, scale, cfg.collect_rows, out=outs, logits=logits[r], lse=lses,
                            workspace=ws_v)

    def select(r):
        if physical:
            lcs.select_topk_physical(logits[r], pl, L, cfg.Hkv, cfg.mode, cfg.top_k, cfg.n_sink, cfg.n_recent,
                                     layers[r], cap=S, indices=idx[r], counts=cnt[r], workspace=ws_s)
        elif scores:
            lcs.select_topk_scores(logits[r], pl, L, cfg.mode, cfg.top_k, cfg.n_sink, cfg.n_recent, cap=S,
                                   indices=idx[r], counts=cnt[r], workspace=ws_s, Hq=Hq)
        else:
            lcs.select_topk(logits[r], pl, L, cfg.Hkv, cfg.mode, cfg.top_k, cfg.n_sink, cfg.n_recent, cap=S,
                            indices=idx[r], counts=cnt[r], workspace=ws_s)

    RF = max(1, refresh_every)
    refresh = [r for r in range(R) if r % RF == 0]       # layers that derive their own sets

    def draft(r, j):
        rs = r - r % RF                                  # reuse layers take the refresh layer's sets
        draft_fn = lcs.sparse_draft_attn_physical if physical else lcs.sparse_draft_attn
        draft_fn(layers[r], qds[j], cfg.mode, idx[rs], cnt[rs], pl, tls[j], max_tl, scale, out=dout, lse=dlse,
                 workspace=ws_d)

    for r in range(R):       # the first iteration's sparse sets
        verify(r)
        select(r)
    torch.cuda.synchronize()

    E = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731
    phase_ms = {"draft": 0.0, "verify": 0.0, "select": 0.0}

    def step():
        ev = []
        e0 = E(); e0.record(); ev.append(("start", e0))
        for j in range(cfg.n_draft):
            for r in range(R):
                draft(r, j)
        e1 = E(); e1.record(); ev.append(("draft", e1))
        for r in range(R):
            verify(r)
        e2 = E(); e2.record(); ev.append(("verify", e2))
        for r in refresh:
            select(r)
        e3 = E(); e3.record(); ev.append(("select", e3))
        return ev

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    events = []
    t0 = time.perf_counter()
    for _ in range(steps):
        events.append(step())
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    for ev in events:
        for (_, a), (name, b) in zip(ev[:-1], ev[1:]):
            phase_ms[name] += a.elapsed_time(b)
    ms_per_step = wall * 1e3 / steps
    t_draft_us = phase_ms["draft"] * 1e3 / (steps * cfg.n_draft * R)
    t_verify_us = phase_ms["verify"] * 1e3 / (steps * R)
    t_select_us = phase_ms["select"] * 1e3 / (steps * len(refresh))
    s_count = int(cnt[0].min().item())
    tail_lens = [cfg.n_q + j + 1 for j in range(cfg.n_draft)]
    vb, sb, db = algorithmic_bytes(cfg, s_count, tail_lens, scores=scores)
    step_bytes = R * (vb + sum(db)) + len(refresh) * sb
    del logits, idx, cnt, ws_v, ws_s, ws_d
    return {"ms_per_step": ms_per_step, "step_bytes": step_bytes, "us": {"verify": t_verify_us,
            "select": t_select_us, "draft_step": t_draft_us},
            "bytes": {"verify": vb, "select": sb, "draft_step": int(sum(db) / len(db))},
            "share": {"verify": phase_ms["verify"], "select": phase_ms["select"], "draft": phase_ms["draft"]},
            "selected": s_count, "R": R, "refresh": len(refresh), "RF": RF}


def kernel_table(cfg, m):
    """Per-call latency, algorithmic bytes and fraction of the 8 TB/s peak."""
    res = {}
    for name in ("verify", "select", "draft_step"):
        us, by = m["us"][name], m["bytes"][name]
        gbs = by / (us * 1e-6) / 1e9
        res[name] = {"us": round(us, 2), "bytes": by, "GB/s": round(gbs, 1),
                     "frac_hbm_peak": round(gbs / HBM_PEAK_GBS, 4)}
    flops_verify = 4 * cfg.B * cfg.Hq * cfg.n_q * (cfg.L + cfg.n_q) * cfg.d
    res["verify"]["TFLOP/s"] = round(flops_verify / (m["us"]["verify"] * 1e-6) / 1e12, 2)
    res["draft_step"]["selected"] = m["selected"]
    return res


# the kernels behind each call, as rocprofv3 names them
CALL_KERNELS = {"verify": "attn_kernel (dense verify) + combine_kernel",
                "select": "score_kernel + collect_kernel + finish_kernel",
                "draft_step": "attn_kernel (shared token list) + combine_kernel"}


def main():
    args = parse()
    if args.oracle_timing:
        oracle_timing()
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported (the multi-GPU "
              "sharding of this path is described in the design notes, not built).", file=sys.stderr)
        sys.exit(2)
    import torch

    from long_context_self_amd import synth

    torch.cuda.set_device(0)
    cfg = synth.CONFIGS[args.config]
    R = args.layers or DEFAULT_LAYERS.get(cfg.name, 4)
    ws = setup_workload(cfg, R, copy_calibration_mib=args.copy_calibration_mib, log=sys.stderr)
    m = measure(ws, args.steps, args.warmup, scores=args.scores, refresh_every=args.refresh_every,
                physical=args.physical)
    variants = {}
    if not args.no_variants and not (args.scores or args.physical or args.refresh_every != 1):
        # the fused variants of the same step on the same inputs (not the headline)
        for name, kw in (("partial_scores", {"scores": True}), ("physical_hand_off", {"physical": True})):
            mv = measure(ws, args.steps, args.warmup, **kw)
            variants[name] = {"ms_per_step": round(mv["ms_per_step"], 4),
                              "value_GB/s": round(mv["step_bytes"] / (mv["ms_per_step"] * 1e-3) / 1e9, 2),
                              "kernels": kernel_table(cfg, mv)}
    del ws
    torch.cuda.empty_cache()
    kern = kernel_table(cfg, m)
    value = m["step_bytes"] / (m["ms_per_step"] * 1e-3) / 1e9
    # the call with the largest share of the step's time carries the roofline
    share = {"verify": m["share"]["verify"], "select": m["share"]["select"], "draft_step": m["share"]["draft"]}
    dom = max(share, key=share.get)
    traffic = None
    if not args.scores and not args.physical and args.refresh_every == 1:
        traffic = traffic_record(cfg.name, dom)
    result = {
        "metric": "draft-step & verify-step attention latency (us), achieved HBM GB/s vs peak",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(m["ms_per_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": cfg.name, "B": cfg.B, "Hq": cfg.Hq, "Hkv": cfg.Hkv, "d": cfg.d, "L": cfg.L,
                   "page_size": cfg.page_size, "n_q": cfg.n_q, "n_draft": cfg.n_draft,
                   "select": f"{cfg.mode} top-{cfg.top_k}+{cfg.n_sink} sink+{cfg.n_recent} recent",
                   "collected": "per-KV-head partial scores" if args.scores else "two logit rows",
                   "hand_off": "physical cache slots" if args.physical else "positions",
                   "refresh_every": m["RF"], "layers": R},
        "kernels": kern,
        "step_share": {k: round(v / sum(share.values()), 4) for k, v in share.items()},
        "gamma_attn": round(m["us"]["draft_step"] / m["us"]["verify"], 4),
        "roofline": {"bound": "hbm", "achieved": kern[dom]["GB/s"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": kern[dom]["frac_hbm_peak"], "traffic": traffic,
                     "kernel": f"{dom}: {CALL_KERNELS[dom]}, per call",
                     "algorithmic_bytes": kern[dom]["bytes"]},
    }
    if variants:
        result["variants"] = variants
    if not args.no_secondary and args.config != SECONDARY_CONFIG:
        c2 = synth.CONFIGS[SECONDARY_CONFIG]
        ws2 = setup_workload(c2, DEFAULT_LAYERS[SECONDARY_CONFIG], log=sys.stderr)
        m2 = measure(ws2, args.steps, args.warmup, scores=args.scores, physical=args.physical)
        del ws2
        result["secondary"] = {"workload": c2.name, "layers": m2["R"], "ms_per_step": round(m2["ms_per_step"], 4),
                               "value_GB/s": round(m2["step_bytes"] / (m2["ms_per_step"] * 1e-3) / 1e9, 2),
                               "kernels": kernel_table(c2, m2)}
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(cfg, args.cpu_seconds)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
