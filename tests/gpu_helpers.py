"""Plumbing for the GPU tests: move seeded numpy inputs to the device and back."""
import math

import numpy as np
import pytest

from long_context_self_amd import synth


def require_gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    from long_context_self_amd import lcs
    lcs.load()           # fails loudly if the library was not built
    return torch, lcs


def bf16_dev(bits: np.ndarray, torch, device="cuda"):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(device)


def i32_dev(a, torch, device="cuda"):
    return torch.from_numpy(np.ascontiguousarray(np.asarray(a, dtype=np.int32))).to(device)


def u64_dev(a, torch, device="cuda"):
    return torch.from_numpy(np.ascontiguousarray(np.asarray(a, dtype=np.uint64)).view(np.int64)).to(device)


def kv_dev(kv: synth.PagedKV, torch, lcs, device="cuda"):
    return lcs.PagedKV(bf16_dev(kv.k, torch, device), bf16_dev(kv.v, torch, device),
                       i32_dev(kv.block_table, torch, device))


def scale_for(d: int) -> float:
    return 1.0 / math.sqrt(d)


def logit_rel_err(g: np.ndarray, o: np.ndarray) -> float:
    """max |g - o| / max(|o|, rms(o over the row)) over the last axis (logit tolerance reading)."""
    o = np.asarray(o, dtype=np.float64)
    g = np.asarray(g, dtype=np.float64)
    if o.size == 0:
        return 0.0       # an empty prefix has no logits to compare
    rms = np.sqrt(np.mean(o * o, axis=-1, keepdims=True))
    den = np.maximum(np.abs(o), rms)
    den = np.where(den > 0, den, 1.0)
    return float(np.max(np.abs(g - o) / den)) if o.size else 0.0
