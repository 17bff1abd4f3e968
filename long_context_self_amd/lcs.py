"""Thin Python binding of liblcs.so (include/lcs.h): argument marshalling only.

Every step of the path runs in the library's HIP kernels; this module only
turns torch tensors into device pointers, sizes workspaces and raises on a
non-OK status.  PyTorch supplies device memory and the current stream.

The library must have been built (``python -m long_context_self_amd._build``
or ``__graft_entry__.build()``); loading fails loudly otherwise.
"""
from __future__ import annotations

import ctypes
import dataclasses
import os
from typing import Optional, Tuple

import torch

from ._build import lib_path

LCS_OK, LCS_E_ARG, LCS_E_SHAPE, LCS_E_WORKSPACE, LCS_E_UNSUPPORTED, LCS_E_HIP = range(6)
SET_MODES = {"shared": 0, "per_kv_head": 1, "block": 2}

STATUS_NAMES = {0: "LCS_OK", 1: "LCS_E_ARG", 2: "LCS_E_SHAPE", 3: "LCS_E_WORKSPACE",
                4: "LCS_E_UNSUPPORTED", 5: "LCS_E_HIP"}


class LcsError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


class PagedKVDesc(ctypes.Structure):
    _fields_ = [("k", ctypes.c_void_p), ("v", ctypes.c_void_p), ("block_table", ctypes.c_void_p),
                ("num_pages", ctypes.c_int32), ("page_size", ctypes.c_int32),
                ("max_pages", ctypes.c_int32), ("Hkv", ctypes.c_int32), ("d", ctypes.c_int32)]


_i32, _i64, _sz, _p, _f = ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_float
_u64 = ctypes.c_uint64
_KV = ctypes.POINTER(PagedKVDesc)

SIGNATURES = {
    "lcs_verify_workspace_bytes": (_sz, [_i32, _i32, _i32, _KV, _i32]),
    "lcs_verify_attn": (_i32, [_KV, _p, _i32, _i32, _i32, _p, _i32, _p, _f, _i32, _i32, _p, _p, _i64,
                              _p, _p, _sz, _p]),
    "lcs_verify_attn_rows": (_i32, [_KV, _p, _i32, _i32, _i32, _p, _i32, _p, _f, _u64, _p, _p, _i64,
                                   _p, _p, _sz, _p]),
    "lcs_verify_attn_scores": (_i32, [_KV, _p, _i32, _i32, _i32, _p, _i32, _p, _f, _i32, _i32, _p, _p,
                                     _i64, _p, _p, _sz, _p]),
    "lcs_select_workspace_bytes": (_sz, [_i32, _i32, _i32, _i32, _i32, _i32]),
    "lcs_select_topk_scores": (_i32, [_p, _i64, _i32, _i32, _p, _i32, _i32, _i32, _i32, _i32, _i32, _p, _p,
                                     _i32, _p, _sz, _p]),
    "lcs_select_topk_rows": (_i32, [_p, _i64, _i32, _i32, _p, _i32, _u64, _i32, _i32, _i32, _p, _i32, _i32,
                                   _i32, _i32, _i32, _i32, _p, _p, _i32, _p, _sz, _p]),
    "lcs_select_topk": (_i32, [_p, _i64, _i32, _i32, _i32, _p, _i32, _i32, _i32, _i32, _i32, _i32,
                              _p, _p, _i32, _p, _sz, _p]),
    "lcs_sparse_workspace_bytes": (_sz, [_i32, _i32, _i32, _KV, _i32, _i32, _i32]),
    "lcs_sparse_draft_attn": (_i32, [_KV, _p, _i32, _i32, _i32, _i32, _p, _p, _i32, _p, _p, _i32, _p,
                                    _f, _p, _p, _p, _sz, _p]),
    "lcs_sparse_draft_attn_noalloc": (_i32, [_KV, _p, _i32, _i32, _i32, _i32, _p, _p, _i32, _p, _p, _i32,
                                            _p, _f, _p, _p, _p]),
    "lcs_select_topk_physical": (_i32, [_p, _i64, _i32, _i32, _i32, _p, _i32, _i32, _i32, _i32, _i32, _KV, _p, _p,
                                       _i32, _p, _sz, _p]),
    "lcs_sparse_draft_attn_physical": (_i32, [_KV, _p, _i32, _i32, _i32, _i32, _p, _p, _i32, _p, _p, _i32, _p,
                                             _f, _p, _p, _p, _sz, _p]),
    "lcs_select_topk_blocks": (_i32, [_p, _i64, _i32, _i32, _i32, _p, _i32, _i32, _i32, _i32, _i32, _i32, _p, _p,
                                     _i32, _p, _sz, _p]),
    "lcs_nsa_compress": (_i32, [_KV, _i32, _p, _i32, _i32, _i32, _p, _p, _i32, _p]),
    "lcs_nsa_plan_bytes": (_sz, [_i32, _i32, _i32, _i32]),
    "lcs_nsa_plan": (_i32, [_KV, _i32, _i32, _p, _p, _i32, _i32, _p, _sz, _p]),
    "lcs_nsa_workspace_bytes": (_sz, [_i32, _i32, _i32, _KV, _i32, _i32, _i32, _i32]),
    "lcs_nsa_attn": (_i32, [_KV, _p, _p, _i32, _i32, _i32, _i32, _p, _i32, _i32, _i32, _p, _sz, _i32, _p, _p, _i32,
                           _p, _p, _f, _p, _p, _p, _sz, _p]),
    "lcs_last_error": (ctypes.c_char_p, []),
    "lcs_version": (ctypes.c_char_p, []),
}

_LIB = None


def load() -> ctypes.CDLL:
    """Load liblcs.so; raises if it has not been built."""
    global _LIB
    if _LIB is None:
        path = lib_path()
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is missing: build it with __graft_entry__.build() "
                               "or python -m long_context_self_amd._build")
        lib = ctypes.CDLL(path)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _LIB = lib
    return _LIB


def _check(status: int) -> None:
    if status != LCS_OK:
        raise LcsError(status, load().lcs_last_error().decode())


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors passed to liblcs must be contiguous")
    return t.data_ptr()


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


@dataclasses.dataclass
class PagedKV:
    """Device-side paged cache: k, v bf16 [num_pages][Hkv][page_size][d]; block_table int32 [B][max_pages]."""
    k: torch.Tensor
    v: torch.Tensor
    block_table: torch.Tensor

    def desc(self) -> PagedKVDesc:
        n, hkv, ps, d = self.k.shape
        return PagedKVDesc(_ptr(self.k), _ptr(self.v), _ptr(self.block_table), n, ps,
                           self.block_table.shape[1], hkv, d)


def _workspace(nbytes: int, device, ws: Optional[torch.Tensor]) -> torch.Tensor:
    if ws is not None and ws.numel() >= nbytes:
        return ws
    return torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)


def verify_workspace_bytes(kv: PagedKV, B: int, n_q: int, Hq: int, max_prefix_len: int) -> int:
    d = kv.desc()
    return load().lcs_verify_workspace_bytes(B, n_q, Hq, ctypes.byref(d), max_prefix_len)


def row_ld(n: int) -> int:
    """Row stride (in floats) for fp32 logit or score rows of n positions: n rounded up to
    64, plus 32.  Rows then start 128 bytes past a multiple of 256 bytes apart, which
    spreads the verify kernel's concurrent row writes over the HBM channels; a
    power-of-two stride makes them collide."""
    return (max(n, 1) + 63) // 64 * 64 + 32


def verify_attn(kv: PagedKV, q: torch.Tensor, prefix_len: torch.Tensor, max_prefix_len: int,
                scale: float, collect_rows: Tuple[int, int], tree_mask: Optional[torch.Tensor] = None,
                out: Optional[torch.Tensor] = None, logits: Optional[torch.Tensor] = None,
                lse: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                with_logits: bool = True):
    """lcs_verify_attn.  q bf16 [B][n_q][Hq][d].  Returns (out, logits, lse)."""
    B, n_q, Hq, d = q.shape
    dev = q.device
    if out is None:
        out = torch.empty((B, n_q, Hq, d), dtype=torch.float32, device=dev)
    if logits is None and with_logits:
        logits = torch.empty((B, Hq, 2, max(max_prefix_len, 1)), dtype=torch.float32, device=dev)
    if lse is None:
        lse = torch.empty((B, n_q, Hq), dtype=torch.float32, device=dev)
    desc = kv.desc()
    need = load().lcs_verify_workspace_bytes(B, n_q, Hq, ctypes.byref(desc), max_prefix_len)
    ws = _workspace(need, dev, workspace)
    ld = logits.shape[-1] if logits is not None else 0
    _check(load().lcs_verify_attn(ctypes.byref(desc), _ptr(q), B, n_q, Hq, _ptr(prefix_len),
                                  max_prefix_len, _ptr(tree_mask), scale, collect_rows[0],
                                  collect_rows[1], _ptr(out), _ptr(logits), ld, _ptr(lse),
                                  ws.data_ptr(), ws.numel(), _stream()))
    return out, logits, lse


def rows_mask(rows) -> int:
    """Bit mask of verifier rows (ascending slots in the collected logits)."""
    m = 0
    for r in rows:
        m |= 1 << int(r)
    return m


def verify_attn_rows(kv: PagedKV, q: torch.Tensor, prefix_len: torch.Tensor, max_prefix_len: int,
                     scale: float, rows, tree_mask: Optional[torch.Tensor] = None,
                     out: Optional[torch.Tensor] = None, logits: Optional[torch.Tensor] = None,
                     lse: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                     with_logits: bool = True):
    """lcs_verify_attn_rows.  rows: the verifier rows to collect (any order; slots are
    ascending).  Returns (out, logits [B][Hq][len(rows)][ld] or None, lse)."""
    B, n_q, Hq, d = q.shape
    dev = q.device
    mask = rows_mask(rows)
    n_c = bin(mask).count("1")
    if out is None:
        out = torch.empty((B, n_q, Hq, d), dtype=torch.float32, device=dev)
    if logits is None and with_logits and n_c > 0:
        logits = torch.empty((B, Hq, n_c, max(max_prefix_len, 1)), dtype=torch.float32, device=dev)
    if lse is None:
        lse = torch.empty((B, n_q, Hq), dtype=torch.float32, device=dev)
    desc = kv.desc()
    need = load().lcs_verify_workspace_bytes(B, n_q, Hq, ctypes.byref(desc), max_prefix_len)
    ws = _workspace(need, dev, workspace)
    ld = logits.shape[-1] if logits is not None else 0
    _check(load().lcs_verify_attn_rows(ctypes.byref(desc), _ptr(q), B, n_q, Hq, _ptr(prefix_len),
                                       max_prefix_len, _ptr(tree_mask), scale, mask, _ptr(out),
                                       _ptr(logits), ld, _ptr(lse), ws.data_ptr(), ws.numel(), _stream()))
    return out, logits, lse


def verify_attn_scores(kv: PagedKV, q: torch.Tensor, prefix_len: torch.Tensor, max_prefix_len: int,
                       scale: float, collect_rows: Tuple[int, int], tree_mask: Optional[torch.Tensor] = None,
                       out: Optional[torch.Tensor] = None, scores: Optional[torch.Tensor] = None,
                       lse: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None):
    """lcs_verify_attn_scores.  Returns (out, scores [B][Hkv][ld], lse)."""
    B, n_q, Hq, d = q.shape
    dev = q.device
    Hkv = kv.k.shape[1]
    if out is None:
        out = torch.empty((B, n_q, Hq, d), dtype=torch.float32, device=dev)
    if scores is None:
        scores = torch.empty((B, Hkv, max(max_prefix_len, 1)), dtype=torch.float32, device=dev)
    if lse is None:
        lse = torch.empty((B, n_q, Hq), dtype=torch.float32, device=dev)
    desc = kv.desc()
    need = load().lcs_verify_workspace_bytes(B, n_q, Hq, ctypes.byref(desc), max_prefix_len)
    ws = _workspace(need, dev, workspace)
    _check(load().lcs_verify_attn_scores(ctypes.byref(desc), _ptr(q), B, n_q, Hq, _ptr(prefix_len),
                                         max_prefix_len, _ptr(tree_mask), scale, collect_rows[0],
                                         collect_rows[1], _ptr(out), _ptr(scores), scores.stride(1), _ptr(lse),
                                         ws.data_ptr(), ws.numel(), _stream()))
    return out, scores, lse


def select_topk_scores(scores: torch.Tensor, prefix_len: torch.Tensor, max_prefix_len: int, mode: str,
                       top_k: int, n_sink: int, n_recent: int, block_size: int = 0, cap: Optional[int] = None,
                       indices: Optional[torch.Tensor] = None, counts: Optional[torch.Tensor] = None,
                       workspace: Optional[torch.Tensor] = None, Hq: Optional[int] = None):
    """lcs_select_topk_scores.  scores fp32 [B][Hkv][ld].  Returns (indices, counts)."""
    B, Hkv = scores.shape[0], scores.shape[1]
    dev = scores.device
    n_sets = 1 if mode == "shared" else Hkv
    if cap is None:
        if mode == "block":
            nb = -(-max_prefix_len // block_size)
            cap = min(nb, -(-n_sink // block_size) + top_k + -(-n_recent // block_size) + 1)
        else:
            cap = min(max_prefix_len, n_sink + top_k + n_recent)
        cap = max(cap, 1)
    if indices is None:
        indices = torch.full((B, n_sets, cap), -1, dtype=torch.int32, device=dev)
    if counts is None:
        counts = torch.zeros((B, n_sets), dtype=torch.int32, device=dev)
    need = load().lcs_select_workspace_bytes(B, Hq or Hkv, Hkv, SET_MODES[mode], max_prefix_len, block_size)
    ws = _workspace(need, dev, workspace)
    _check(load().lcs_select_topk_scores(_ptr(scores), scores.stride(1), B, Hkv, _ptr(prefix_len),
                                         max_prefix_len, SET_MODES[mode], top_k, n_sink, n_recent, block_size,
                                         _ptr(indices), _ptr(counts), cap, ws.data_ptr(), ws.numel(), _stream()))
    return indices, counts


def select_workspace_bytes(B: int, Hq: int, Hkv: int, mode: str, max_prefix_len: int,
                           block_size: int = 0) -> int:
    return load().lcs_select_workspace_bytes(B, Hq, Hkv, SET_MODES[mode], max_prefix_len, block_size)


def select_topk(logits: torch.Tensor, prefix_len: torch.Tensor, max_prefix_len: int, Hkv: int,
                mode: str, top_k: int, n_sink: int, n_recent: int, block_size: int = 0,
                cap: Optional[int] = None, indices: Optional[torch.Tensor] = None,
                counts: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None):
    """lcs_select_topk.  logits fp32 [B][Hq][2][ld].  Returns (indices [B][n_sets][cap], counts [B][n_sets])."""
    B, Hq = logits.shape[0], logits.shape[1]
    dev = logits.device
    n_sets = 1 if mode == "shared" else Hkv
    if cap is None:
        if mode == "block":
            nb = -(-max_prefix_len // block_size)
            cap = min(nb, -(-n_sink // block_size) + top_k + -(-n_recent // block_size) + 1)
        else:
            cap = min(max_prefix_len, n_sink + top_k + n_recent)
        cap = max(cap, 1)
    if indices is None:
        indices = torch.full((B, n_sets, cap), -1, dtype=torch.int32, device=dev)
    if counts is None:
        counts = torch.zeros((B, n_sets), dtype=torch.int32, device=dev)
    need = load().lcs_select_workspace_bytes(B, Hq, Hkv, SET_MODES[mode], max_prefix_len, block_size)
    ws = _workspace(need, dev, workspace)
    _check(load().lcs_select_topk(_ptr(logits), logits.stride(2), B, Hq, Hkv, _ptr(prefix_len),
                                  max_prefix_len, SET_MODES[mode], top_k, n_sink, n_recent, block_size,
                                  _ptr(indices), _ptr(counts), cap, ws.data_ptr(), ws.numel(),
                                  _stream()))
    return indices, counts


SCORE_KINDS = {"logits": 0, "weights": 1}


def select_topk_rows(logits: torch.Tensor, prefix_len: torch.Tensor, max_prefix_len: int, Hkv: int,
                     mode: str, top_k: int, n_sink: int, n_recent: int, score: str = "logits",
                     lse: Optional[torch.Tensor] = None, rows=None, block_size: int = 0,
                     cap: Optional[int] = None, indices: Optional[torch.Tensor] = None,
                     counts: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None):
    """lcs_select_topk_rows.  logits fp32 [B][Hq][n_rows][ld]; score "logits" or
    "weights" (the latter needs lse [B][n_q][Hq] and the collected rows)."""
    B, Hq, n_rows = logits.shape[0], logits.shape[1], logits.shape[2]
    dev = logits.device
    n_sets = 1 if mode == "shared" else Hkv
    if cap is None:
        if mode == "block":
            nb = -(-max_prefix_len // block_size)
            cap = min(nb, -(-n_sink // block_size) + top_k + -(-n_recent // block_size) + 1)
        else:
            cap = min(max_prefix_len, n_sink + top_k + n_recent)
        cap = max(cap, 1)
    if indices is None:
        indices = torch.full((B, n_sets, cap), -1, dtype=torch.int32, device=dev)
    if counts is None:
        counts = torch.zeros((B, n_sets), dtype=torch.int32, device=dev)
    n_q = lse.shape[1] if lse is not None else 0
    mask = rows_mask(rows) if rows is not None else 0
    need = load().lcs_select_workspace_bytes(B, Hq, Hkv, SET_MODES[mode], max_prefix_len, block_size)
    ws = _workspace(need, dev, workspace)
    _check(load().lcs_select_topk_rows(_ptr(logits), logits.stride(2), n_rows, SCORE_KINDS[score], _ptr(lse),
                                       n_q, mask, B, Hq, Hkv, _ptr(prefix_len), max_prefix_len,
                                       SET_MODES[mode], top_k, n_sink, n_recent, block_size, _ptr(indices),
                                       _ptr(counts), cap, ws.data_ptr(), ws.numel(), _stream()))
    return indices, counts


def sparse_workspace_bytes(kv: PagedKV, B: int, n_q: int, Hq: int, mode: str, cap: int,
                           max_tail_len: int) -> int:
    d = kv.desc()
    return load().lcs_sparse_workspace_bytes(B, n_q, Hq, ctypes.byref(d), SET_MODES[mode], cap, max_tail_len)


def sparse_draft_attn(kv: PagedKV, q: torch.Tensor, mode: str, indices: torch.Tensor,
                      counts: torch.Tensor, tail_begin: torch.Tensor, tail_len: torch.Tensor,
                      max_tail_len: int, scale: float, tail_mask: Optional[torch.Tensor] = None,
                      out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                      workspace: Optional[torch.Tensor] = None):
    """lcs_sparse_draft_attn.  q bf16 [B][n_q][Hq][d].  Returns (out, lse)."""
    B, n_q, Hq, d = q.shape
    dev = q.device
    cap = indices.shape[-1]
    if out is None:
        out = torch.empty((B, n_q, Hq, d), dtype=torch.float32, device=dev)
    if lse is None:
        lse = torch.empty((B, n_q, Hq), dtype=torch.float32, device=dev)
    desc = kv.desc()
    need = load().lcs_sparse_workspace_bytes(B, n_q, Hq, ctypes.byref(desc), SET_MODES[mode], cap,
                                             max_tail_len)
    ws = _workspace(need, dev, workspace)
    _check(load().lcs_sparse_draft_attn(ctypes.byref(desc), _ptr(q), B, n_q, Hq, SET_MODES[mode],
                                        _ptr(indices), _ptr(counts), cap, _ptr(tail_begin),
                                        _ptr(tail_len), max_tail_len, _ptr(tail_mask), scale,
                                        _ptr(out), _ptr(lse), ws.data_ptr(), ws.numel(), _stream()))
    return out, lse


def select_topk_physical(logits: torch.Tensor, prefix_len: torch.Tensor, max_prefix_len: int, Hkv: int,
                         mode: str, top_k: int, n_sink: int, n_recent: int, kv: PagedKV,
                         cap: Optional[int] = None, indices: Optional[torch.Tensor] = None,
                         counts: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None):
    """lcs_select_topk_physical: the selected positions as physical cache slots through
    kv's block table.  Returns (indices [B][n_sets][cap], counts [B][n_sets])."""
    B, Hq = logits.shape[0], logits.shape[1]
    dev = logits.device
    n_sets = 1 if mode == "shared" else Hkv
    if cap is None:
        cap = max(1, min(max_prefix_len, n_sink + top_k + n_recent))
    if indices is None:
        indices = torch.full((B, n_sets, cap), -1, dtype=torch.int32, device=dev)
    if counts is None:
        counts = torch.zeros((B, n_sets), dtype=torch.int32, device=dev)
    need = load().lcs_select_workspace_bytes(B, Hq, Hkv, SET_MODES[mode], max_prefix_len, 0)
    ws = _workspace(need, dev, workspace)
    desc = kv.desc()
    _check(load().lcs_select_topk_physical(_ptr(logits), logits.stride(2), B, Hq, Hkv, _ptr(prefix_len),
                                           max_prefix_len, SET_MODES[mode], top_k, n_sink, n_recent,
                                           ctypes.byref(desc), _ptr(indices), _ptr(counts), cap, ws.data_ptr(),
                                           ws.numel(), _stream()))
    return indices, counts


def sparse_draft_attn_physical(kv: PagedKV, q: torch.Tensor, mode: str, indices: torch.Tensor,
                               counts: torch.Tensor, tail_begin: torch.Tensor, tail_len: torch.Tensor,
                               max_tail_len: int, scale: float, tail_mask: Optional[torch.Tensor] = None,
                               out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                               workspace: Optional[torch.Tensor] = None):
    """lcs_sparse_draft_attn_physical: lists of physical cache slots.  Returns (out, lse)."""
    B, n_q, Hq, d = q.shape
    dev = q.device
    cap = indices.shape[-1]
    if out is None:
        out = torch.empty((B, n_q, Hq, d), dtype=torch.float32, device=dev)
    if lse is None:
        lse = torch.empty((B, n_q, Hq), dtype=torch.float32, device=dev)
    desc = kv.desc()
    need = load().lcs_sparse_workspace_bytes(B, n_q, Hq, ctypes.byref(desc), SET_MODES[mode], cap, max_tail_len)
    ws = _workspace(need, dev, workspace)
    _check(load().lcs_sparse_draft_attn_physical(ctypes.byref(desc), _ptr(q), B, n_q, Hq, SET_MODES[mode],
                                                 _ptr(indices), _ptr(counts), cap, _ptr(tail_begin),
                                                 _ptr(tail_len), max_tail_len, _ptr(tail_mask), scale,
                                                 _ptr(out), _ptr(lse), ws.data_ptr(), ws.numel(), _stream()))
    return out, lse


BLOCK_SCORES = {"max": 0, "lse": 1}
GROUP_MODES = {"exact": 0, "approximate": 1}


def select_topk_blocks(logits: torch.Tensor, prefix_len: torch.Tensor, max_prefix_len: int, Hkv: int,
                       block_score: str, top_k: int, n_sink: int, n_recent: int, block_size: int,
                       cap: Optional[int] = None, indices: Optional[torch.Tensor] = None,
                       counts: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None):
    """lcs_select_topk_blocks: per-KV-head block sets scored by "max" or "lse".
    Returns (indices [B][Hkv][cap], counts [B][Hkv])."""
    B, Hq = logits.shape[0], logits.shape[1]
    dev = logits.device
    if cap is None:
        nb = -(-max_prefix_len // block_size)
        cap = max(1, min(nb, -(-n_sink // block_size) + top_k + -(-n_recent // block_size) + 1))
    if indices is None:
        indices = torch.full((B, Hkv, cap), -1, dtype=torch.int32, device=dev)
    if counts is None:
        counts = torch.zeros((B, Hkv), dtype=torch.int32, device=dev)
    need = load().lcs_select_workspace_bytes(B, Hq, Hkv, SET_MODES["block"], max_prefix_len, block_size)
    ws = _workspace(need, dev, workspace)
    _check(load().lcs_select_topk_blocks(_ptr(logits), logits.stride(2), B, Hq, Hkv, _ptr(prefix_len),
                                         max_prefix_len, BLOCK_SCORES[block_score], top_k, n_sink, n_recent,
                                         block_size, _ptr(indices), _ptr(counts), cap, ws.data_ptr(), ws.numel(),
                                         _stream()))
    return indices, counts


def nsa_compress(kv: PagedKV, prefix_len: torch.Tensor, max_prefix_len: int, cmp_len: int, cmp_stride: int,
                 max_cmp: int, k_cmp: Optional[torch.Tensor] = None, v_cmp: Optional[torch.Tensor] = None):
    """lcs_nsa_compress.  Returns the compressed cache (k_cmp, v_cmp) bf16 [B][Hkv][max_cmp][d]."""
    B = prefix_len.shape[0]
    _, Hkv, _, d = kv.k.shape
    dev = kv.k.device
    if k_cmp is None:
        k_cmp = torch.empty((B, Hkv, max_cmp, d), dtype=torch.bfloat16, device=dev)
    if v_cmp is None:
        v_cmp = torch.empty((B, Hkv, max_cmp, d), dtype=torch.bfloat16, device=dev)
    desc = kv.desc()
    _check(load().lcs_nsa_compress(ctypes.byref(desc), B, _ptr(prefix_len), max_prefix_len, cmp_len, cmp_stride,
                                   _ptr(k_cmp), _ptr(v_cmp), max_cmp, _stream()))
    return k_cmp, v_cmp


def nsa_plan(kv: PagedKV, indices: torch.Tensor, counts: torch.Tensor, group: str = "exact",
             plan: Optional[torch.Tensor] = None) -> torch.Tensor:
    """lcs_nsa_plan: block-union plan of indices [B][n_q][Hkv][cap].  Returns the plan buffer."""
    B, n_q, Hkv, cap = indices.shape
    need = load().lcs_nsa_plan_bytes(B, n_q, Hkv, cap)
    if plan is None or plan.numel() < need:
        plan = torch.empty(max(need, 256), dtype=torch.uint8, device=indices.device)
    desc = kv.desc()
    _check(load().lcs_nsa_plan(ctypes.byref(desc), B, n_q, _ptr(indices), _ptr(counts), cap, GROUP_MODES[group],
                               _ptr(plan), plan.numel(), _stream()))
    return plan


def nsa_workspace_bytes(kv: PagedKV, B: int, n_q: int, Hq: int, cap: int, max_tail_len: int, max_cmp: int,
                        window: int) -> int:
    d = kv.desc()
    return load().lcs_nsa_workspace_bytes(B, n_q, Hq, ctypes.byref(d), cap, max_tail_len, max_cmp, window)


def nsa_attn(kv: PagedKV, k_cmp: torch.Tensor, v_cmp: torch.Tensor, cmp_len: int, cmp_stride: int, window: int,
             q: torch.Tensor, plan: torch.Tensor, cap: int, tail_begin: torch.Tensor, tail_len: torch.Tensor,
             max_tail_len: int, gates: torch.Tensor, scale: float, tail_mask: Optional[torch.Tensor] = None,
             out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
             workspace: Optional[torch.Tensor] = None):
    """lcs_nsa_attn: gated compression / selection / window attention of q bf16 [B][n_q][Hq][d].
    Returns (out [B][n_q][Hq][d], lse [B][n_q][Hq][3])."""
    B, n_q, Hq, d = q.shape
    dev = q.device
    max_cmp = k_cmp.shape[2]
    if out is None:
        out = torch.empty((B, n_q, Hq, d), dtype=torch.float32, device=dev)
    if lse is None:
        lse = torch.empty((B, n_q, Hq, 3), dtype=torch.float32, device=dev)
    desc = kv.desc()
    need = load().lcs_nsa_workspace_bytes(B, n_q, Hq, ctypes.byref(desc), cap, max_tail_len, max_cmp, window)
    ws = _workspace(need, dev, workspace)
    _check(load().lcs_nsa_attn(ctypes.byref(desc), _ptr(k_cmp), _ptr(v_cmp), max_cmp, cmp_len, cmp_stride, window,
                               _ptr(q), B, n_q, Hq, _ptr(plan), plan.numel(), cap, _ptr(tail_begin), _ptr(tail_len),
                               max_tail_len, _ptr(tail_mask), _ptr(gates), scale, _ptr(out), _ptr(lse),
                               ws.data_ptr(), ws.numel(), _stream()))
    return out, lse


def sparse_draft_attn_noalloc(kv: PagedKV, q: torch.Tensor, mode: str, indices: torch.Tensor,
                              counts: torch.Tensor, tail_begin: torch.Tensor, tail_len: torch.Tensor,
                              max_tail_len: int, scale: float, tail_mask: Optional[torch.Tensor] = None,
                              out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None):
    """lcs_sparse_draft_attn_noalloc: the library's static device scratch instead of a
    workspace (out and lse must be passed in to allocate nothing).  Returns (out, lse)."""
    B, n_q, Hq, d = q.shape
    dev = q.device
    cap = indices.shape[-1]
    if out is None:
        out = torch.empty((B, n_q, Hq, d), dtype=torch.float32, device=dev)
    desc = kv.desc()
    _check(load().lcs_sparse_draft_attn_noalloc(ctypes.byref(desc), _ptr(q), B, n_q, Hq, SET_MODES[mode],
                                                _ptr(indices), _ptr(counts), cap, _ptr(tail_begin),
                                                _ptr(tail_len), max_tail_len, _ptr(tail_mask), scale,
                                                _ptr(out), _ptr(lse), _stream()))
    return out, lse


def version() -> str:
    return load().lcs_version().decode()
