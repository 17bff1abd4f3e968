"""Forward latency of a random-weight transformer stack whose attention is the
library's verification call, against the draft length (timing only).

SSV page, Figure 7: forward latency against the draft length on a Llama3-1B
backbone at 32K context, with the attention layers replaced by NSA sparse
verification; Figure 10 caption: draft lengths 4 and 64.  No trained weights
exist here, so acceptance is not measured: the weights are seeded random, which
changes no timing.

One verification forward of n_q = gamma tree nodes (batch 1), per layer:
  RMSNorm -> QKV projection -> the n_q new K/V rows written into the layer's paged
  cache at positions L .. L + n_q - 1 -> attention of the n_q rows over the cache
  -> output projection + residual -> RMSNorm -> SwiGLU MLP + residual.
Attention is either dense verification (lcs_verify_attn, the n_q rows over every
cached position, two logit rows collected) or NSA sparse verification
(lcs_nsa_attn: compression, per-row selected blocks merged into one union, and the
sliding window, gated per head by a sigmoid of a gate projection).  The projections
and the MLP are plain library GEMMs (torch.matmul); RMSNorm, SiLU, the sigmoid and
the cache writes are torch element-wise operations.  Rotary embeddings are left out:
with random weights they change no timing of the attention path.  Each forward is
captured once in a HIP graph and replayed for timing (eager launches of ~15 small
operations per layer are bound by host dispatch); every replay is checked against
the eager forward.

    python -m long_context_self_amd.experiments layer-stack [--layers 16] [--context 32768]
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np


@dataclasses.dataclass(frozen=True)
class StackShape:
    layers: int = 16          # Llama-3.2-1B: 16 layers, hidden 2048, 32 / 8 heads of 64, MLP 8192
    hidden: int = 2048
    Hq: int = 32
    Hkv: int = 8
    d: int = 64
    mlp: int = 8192
    context: int = 32768
    page_size: int = 64       # one NSA selection block per page
    blocks_per_row: int = 16
    core_blocks: int = 10
    cmp_len: int = 32
    cmp_stride: int = 16
    window: int = 512


def _tree_masks(n_q: int) -> np.ndarray:
    """Two chains hanging off the last committed token (one chain for a single node)."""
    from . import synth
    br = 2 if n_q % 2 == 0 and n_q > 1 else 1
    return synth.tree_tail_masks(n_q, br)


def run(shape: StackShape, gammas=(1, 2, 4, 8, 16, 32, 64), iters: int = 10, warmup: int = 3,
        seed: int = 0, log=None) -> dict:
    import torch

    from . import lcs, synth

    dev = "cuda"
    g = torch.Generator(device=dev)
    g.manual_seed(seed)
    S = shape
    G = S.Hq // S.Hkv
    scale = 1.0 / math.sqrt(S.d)
    max_q = max(gammas)
    L = S.context
    n_tok = L + max_q
    pages = (n_tok + S.page_size - 1) // S.page_size

    def randn(*shp, std=1.0, dtype=torch.bfloat16):
        return (torch.randn(*shp, generator=g, device=dev, dtype=torch.float32) * std).to(dtype)

    # weights (bf16, seeded random, scaled like an initialised model)
    w = []
    for _ in range(S.layers):
        w.append({
            "qkv": randn(S.hidden, (S.Hq + 2 * S.Hkv) * S.d, std=S.hidden ** -0.5),
            "o": randn(S.Hq * S.d, S.hidden, std=(S.Hq * S.d) ** -0.5),
            "gate": randn(S.hidden, 3 * S.Hq, std=S.hidden ** -0.5),
            "up": randn(S.hidden, 2 * S.mlp, std=S.hidden ** -0.5),
            "down": randn(S.mlp, S.hidden, std=S.mlp ** -0.5),
        })
    # per-layer paged caches holding the prefix; pages in a seeded random order
    perm = torch.randperm(pages, generator=torch.Generator().manual_seed(seed)).to(torch.int32)
    bt = perm.view(1, pages).to(dev)
    caches = [lcs.PagedKV(randn(pages, S.Hkv, S.page_size, S.d), randn(pages, S.Hkv, S.page_size, S.d), bt)
              for _ in range(S.layers)]
    prefix = torch.tensor([L], dtype=torch.int32, device=dev)
    # NSA side inputs: compressed caches (the prefix is fixed while timing), per-row block sets
    max_cmp = (L - S.cmp_len) // S.cmp_stride + 1
    comp = [lcs.nsa_compress(c, prefix, L, S.cmp_len, S.cmp_stride, max_cmp) for c in caches]
    n_blocks = L // S.page_size
    rows_of = {}
    for n_q in gammas:
        cfg = synth.Config("stack", B=1, Hq=S.Hq, Hkv=S.Hkv, d=S.d, L=L, page_size=S.page_size, n_q=n_q,
                           n_draft=0, top_k=S.blocks_per_row, n_sink=0, n_recent=0, mode="block", crit_frac=0.0,
                           blocks_per_row=S.blocks_per_row, core_blocks=S.core_blocks)
        sets = synth.make_block_sets(cfg, n_blocks, seed=seed) if S.core_blocks + n_q * (
            S.blocks_per_row - S.core_blocks) <= n_blocks else None
        pos = torch.arange(L, L + n_q, device=dev)
        rows_of[n_q] = {
            "page": bt[0, (pos // S.page_size).long()].long(), "slot": (pos % S.page_size).long(),
            "mask": torch.from_numpy(_tree_masks(n_q).view(np.int64)).to(dev).view(1, n_q),
            "sets": torch.from_numpy(sets).to(dev) if sets is not None else None,
            "tl": torch.tensor([n_q], dtype=torch.int32, device=dev),
        }

    def rms(x):
        return x * torch.rsqrt((x.float() * x.float()).mean(-1, keepdim=True) + 1e-5).to(x.dtype)

    res = {"shape": dataclasses.asdict(S), "points": {}}
    for n_q in gammas:
        rq = rows_of[n_q]
        plan = lcs.nsa_plan(caches[0], rq["sets"], torch.full((1, n_q, S.Hkv), S.blocks_per_row, dtype=torch.int32,
                                                             device=dev)) if rq["sets"] is not None else None
        ws_v = torch.empty(lcs.verify_workspace_bytes(caches[0], 1, n_q, S.Hq, L), dtype=torch.uint8, device=dev)
        ws_n = torch.empty(lcs.nsa_workspace_bytes(caches[0], 1, n_q, S.Hq, S.blocks_per_row, n_q, max_cmp,
                                                   S.window), dtype=torch.uint8, device=dev)
        logits = torch.empty((1, S.Hq, 2, lcs.row_ld(L)), dtype=torch.float32, device=dev)
        out = torch.empty((1, n_q, S.Hq, S.d), dtype=torch.float32, device=dev)
        x0 = randn(n_q, S.hidden)

        def forward(kind):
            x = x0
            for li in range(S.layers):
                W = w[li]
                h = rms(x)
                qkv = h @ W["qkv"]
                q = qkv[:, :S.Hq * S.d].reshape(1, n_q, S.Hq, S.d).contiguous()
                k = qkv[:, S.Hq * S.d:(S.Hq + S.Hkv) * S.d].reshape(n_q, S.Hkv, S.d)
                v = qkv[:, (S.Hq + S.Hkv) * S.d:].reshape(n_q, S.Hkv, S.d)
                c = caches[li]
                c.k[rq["page"], :, rq["slot"], :] = k
                c.v[rq["page"], :, rq["slot"], :] = v
                if kind == "dense":
                    lcs.verify_attn(c, q, prefix, L, scale, (0, n_q - 1), tree_mask=rq["mask"], out=out,
                                    logits=logits, workspace=ws_v)
                else:
                    gates = torch.sigmoid((h @ W["gate"]).float()).reshape(1, n_q, S.Hq, 3).contiguous()
                    lcs.nsa_attn(c, comp[li][0], comp[li][1], S.cmp_len, S.cmp_stride, S.window, q, plan,
                                 S.blocks_per_row, prefix, rq["tl"], n_q, gates, scale, tail_mask=rq["mask"],
                                 out=out, workspace=ws_n)
                x = x + out.to(torch.bfloat16).reshape(n_q, S.Hq * S.d) @ W["o"]
                h = rms(x)
                gu = h @ W["up"]
                x = x + (torch.nn.functional.silu(gu[:, :S.mlp]) * gu[:, S.mlp:]) @ W["down"]
            return x

        point = {}
        for kind in ("dense", "nsa"):
            if kind == "nsa" and plan is None:
                continue
            # eager reference, then the whole forward captured in a HIP graph and replayed:
            # eagerly, the ~15 launches per layer are bound by host dispatch, not the GPU
            side = torch.cuda.Stream()
            side.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(side):
                for _ in range(warmup):
                    ref = forward(kind)
            torch.cuda.current_stream().wait_stream(side)
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            ref = forward(kind)
            e1.record()
            torch.cuda.synchronize()
            point[f"{kind}_eager_ms"] = e0.elapsed_time(e1)
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph):
                y = forward(kind)
            times = []
            for _ in range(iters):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                graph.replay()
                e1.record()
                torch.cuda.synchronize()
                times.append(e0.elapsed_time(e1))
                # every replay reproduces the eager forward
                assert bool(torch.isfinite(y.float()).all())
                assert float((y.float() - ref.float()).abs().max()) <= 1e-2 * max(1.0, float(ref.float().abs().max()))
            point[f"{kind}_ms"] = float(np.median(times))
            del graph
        res["points"][str(n_q)] = point
        if log is not None:
            print(f"gamma {n_q}: {point}", file=log, flush=True)
    return res
