"""Algorithmic bytes of each call: what the method must move, nothing it avoids.

bf16 counts 2 bytes, fp32 and int32 4.  These are the denominators of every GB/s
figure the benchmark and the measurements report (8 TB/s HBM is the peak line).
"""
from __future__ import annotations

HBM_PEAK_GBS = 8000.0


def verify_bytes(cfg, scores: bool = False) -> int:
    """K and V of every cached position, Q, O and lse, and the collected side output:
    two fp32 logit rows per query head, or one partial-score row per KV head."""
    B, Hq, Hkv, d, L, n_q = cfg.B, cfg.Hq, cfg.Hkv, cfg.d, cfg.L, cfg.n_q
    collected = 4 * B * Hkv * L if scores else 8 * B * Hq * L
    return (4 * B * Hkv * d * (L + n_q) + 2 * B * n_q * Hq * d + 4 * B * n_q * Hq * d + 4 * B * n_q * Hq
            + collected)


def select_bytes(cfg, S: int, scores: bool = False) -> int:
    """The collected rows read once, and the index lists and counts written."""
    B, Hq, Hkv, L = cfg.B, cfg.Hq, cfg.Hkv, cfg.L
    n_sets = 1 if cfg.mode == "shared" else Hkv
    collected = 4 * B * Hkv * L if scores else 8 * B * Hq * L
    return collected + 4 * B * n_sets * S + 4 * B * n_sets


def draft_bytes(cfg, S: int, tail_len: int) -> int:
    """The selected K and V rows of every KV head plus the tail, the index list, Q, O, lse."""
    B, Hq, Hkv, d = cfg.B, cfg.Hq, cfg.Hkv, cfg.d
    n_sets = 1 if cfg.mode == "shared" else Hkv
    return (4 * B * Hkv * d * (S + tail_len) + 4 * B * n_sets * S + 2 * B * Hq * d + 4 * B * Hq * d
            + 4 * B * Hq)


def nsa_bytes(cfg, union_blocks: int, max_cmp: int) -> int:
    """NSA sparse verification of the n_q rows: the compressed K/V of every compressed
    block, the K/V of the union blocks (union_blocks summed over (b, g)), the window's
    prefix positions and the tail once per branch that reads them, Q, the gates, O."""
    B, Hq, Hkv, d, n_q, P = cfg.B, cfg.Hq, cfg.Hkv, cfg.d, cfg.n_q, cfg.page_size
    win = min(cfg.window, cfg.L)
    kv_rows = B * Hkv * max_cmp + union_blocks * P + B * Hkv * (win + 2 * n_q)
    return 4 * d * kv_rows + 2 * B * n_q * Hq * d + 4 * B * n_q * Hq * 3 + 4 * B * n_q * Hq * d
