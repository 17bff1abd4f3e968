"""Algorithmic bytes per call (the denominators of every GB/s and roofline figure),
derived independently from the sizes of the arrays a call must touch, and the per-call
figures quoted for the workloads."""
import numpy as np
import pytest

from long_context_self_amd import metrics, synth


def _nbytes(shape, dtype):
    return int(np.prod(shape)) * np.dtype(dtype).itemsize


@pytest.mark.parametrize("name", ["tiny", "llama8b_32k", "qwen14b_64k", "stress_128k"])
def test_verify_bytes_from_array_sizes(name):
    c = synth.CONFIGS[name]
    kv_rows = _nbytes((c.B, c.Hkv, c.L + c.n_q, c.d), np.float16)       # bf16 K rows read
    want = (2 * kv_rows                                                  # K and V
            + _nbytes((c.B, c.n_q, c.Hq, c.d), np.float16)              # q (bf16)
            + _nbytes((c.B, c.n_q, c.Hq, c.d), np.float32)              # out
            + _nbytes((c.B, c.n_q, c.Hq), np.float32)                   # lse
            + _nbytes((c.B, c.Hq, 2, c.L), np.float32))                 # two collected rows
    assert metrics.verify_bytes(c) == want
    scores = want - _nbytes((c.B, c.Hq, 2, c.L), np.float32) + _nbytes((c.B, c.Hkv, c.L), np.float32)
    assert metrics.verify_bytes(c, scores=True) == scores


@pytest.mark.parametrize("name", ["tiny", "llama8b_32k", "qwen14b_64k", "stress_128k"])
def test_select_and_draft_bytes_from_array_sizes(name):
    c = synth.CONFIGS[name]
    S = c.n_sink + c.top_k + c.n_recent
    n_sets = 1 if c.mode == "shared" else c.Hkv
    sel = (_nbytes((c.B, c.Hq, 2, c.L), np.float32) + _nbytes((c.B, n_sets, S), np.int32)
           + _nbytes((c.B, n_sets), np.int32))
    assert metrics.select_bytes(c, S) == sel
    tail = c.n_q + 1
    draft = (2 * _nbytes((c.B, c.Hkv, S + tail, c.d), np.float16)        # selected + tail K and V
             + _nbytes((c.B, n_sets, S), np.int32)                      # index lists
             + _nbytes((c.B, 1, c.Hq, c.d), np.float16)                 # q
             + _nbytes((c.B, 1, c.Hq, c.d), np.float32)                 # out
             + _nbytes((c.B, 1, c.Hq), np.float32))                     # lse
    assert metrics.draft_bytes(c, S, tail) == draft


def test_quoted_workload_figures():
    """The per-call byte counts the measurements are quoted against."""
    c2, c5 = synth.CONFIGS["llama8b_32k"], synth.CONFIGS["stress_128k"]
    assert metrics.verify_bytes(c2) == 142865536              # 142.9 MB
    assert metrics.select_bytes(c2, 2116) == 8397076           # 8.4 MB
    assert metrics.draft_bytes(c2, 2116, 10) == 8741264        # first draft step, 8.74 MB
    assert metrics.verify_bytes(c5) == 4565476352              # 4565.5 MB
    assert metrics.select_bytes(c5, 4164) == 268568736         # 268.6 MB
    # the roofline ceiling the fractions use: MI355X HBM3E, 8 TB/s
    assert metrics.HBM_PEAK_GBS == 8000.0
