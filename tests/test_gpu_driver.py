"""The speculative-iteration driver runs verify -> select -> k draft steps with drift
through the library, and the selection keeps finding the planted critical keys."""
import math

import pytest

from long_context_self_amd import synth

from gpu_helpers import require_gpu

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("mode,scores", [("shared", False), ("per_kv_head", False), ("shared", True)])
def test_driver_loop_with_drift(mode, scores):
    require_gpu()
    from long_context_self_amd import driver
    cfg = synth.CONFIGS["llama8b_32k"].with_(L=8192, top_k=512, crit_frac=0.01, mode=mode)
    res = driver.run(cfg, iters=6, drift=0.1, seed=1, scores=scores)
    med = res["median"]
    for key in ("verify_us", "select_us", "draft_us", "iter_us"):
        assert math.isfinite(med[key]) and med[key] > 0
    assert med["moved_rows"] > 0
    # a set chosen blindly would hold budget / L of the critical keys; the logit-guided
    # set must do clearly better, before and after the keys drift
    blind = (cfg.n_sink + cfg.top_k + cfg.n_recent) / cfg.L
    print(f"{mode}: recall first {res['recall_first']:.3f} last {res['recall_last']:.3f} (blind {blind:.3f})")
    assert res["recall_first"] > 2 * blind and res["recall_last"] > 2 * blind


def test_experiments_overlap_and_collect_overhead():
    """The scoring-variant measurements run end to end: the all-row selection overlaps
    itself fully, every variant beats a blind set on the planted keys, and verify with
    all rows collected writes more than with none."""
    require_gpu()
    from long_context_self_amd import experiments
    cfg = synth.CONFIGS["llama8b_32k"].with_(L=8192, top_k=512, crit_frac=0.01)
    res = experiments.overlap(cfg, seed=2)
    v = res["variants"]
    assert v["all_rows_logits"]["overlap_with_all_rows"] == 1.0
    for name, r in v.items():
        print(name, r["overlap_with_all_rows"], r["critical_recall"])
        assert 0.0 <= r["overlap_with_all_rows"] <= 1.0
        assert r["critical_recall"] > 2 * res["blind_recall"]
    co = experiments.collect_overhead(cfg, replicas=2, iters=2)
    pts = co["points"]
    assert set(pts) == {"0", "1", "2", "half", "all"}
    assert all(p["verify_us"] > 0 for p in pts.values())
    assert pts["all"]["logit_bytes_over_kv"] > pts["2"]["logit_bytes_over_kv"] > 0


@pytest.mark.parametrize("mode", ["shared", "per_kv_head"])
def test_driver_iteration_after_drift_matches_oracle(mode):
    """Several drift iterations, then the last one checked call by call: the device K
    cache equals the host cache the drift rewrote (bit for bit), verify's output and
    collected rows match the fp64 oracle on the drifted cache, select is bit-exact on
    the GPU's own rows and overlaps the oracle's selection, and the last draft step
    matches the oracle over the GPU's set plus the tail."""
    require_gpu()
    import numpy as np

    from long_context_self_amd import driver
    from oracle import attention as oa
    from oracle import select as osel
    from gpu_helpers import logit_rel_err, scale_for

    cfg = synth.CONFIGS["llama8b_32k"].with_(B=2, L=4096, top_k=256, crit_frac=0.02, mode=mode)
    res = driver.run(cfg, iters=3, drift=0.1, seed=4, keep_last=True)
    last = res["last"]
    kv = last["kv"]
    assert res["median"]["moved_rows"] > 0
    # the device-side scatter of the drifted K rows reproduces the host cache exactly
    assert np.array_equal(last["k_after_dev"], last["k_after_host"])
    # the last iteration's calls ran on the cache before its own drift
    scale = scale_for(cfg.d)
    o_out, o_lg, _ = oa.verify_attn(last["q"], last["k_before"], kv.v, kv.block_table, kv.prefix_len,
                                    cfg.page_size, scale)
    assert float(np.max(np.abs(last["out"] - o_out))) <= 1e-2
    for b in range(cfg.B):
        L = int(kv.prefix_len[b])
        assert logit_rel_err(last["logits"][b, :, :, :L], o_lg[b, :, :, :L]) <= 1e-3
    n_sets = 1 if mode == "shared" else cfg.Hkv
    ref32 = osel.select(last["logits"], kv.prefix_len, cfg.Hkv, mode, cfg.top_k, cfg.n_sink, cfg.n_recent,
                        precision="f32")
    ref64 = osel.select(o_lg, kv.prefix_len, cfg.Hkv, mode, cfg.top_k, cfg.n_sink, cfg.n_recent)
    for b in range(cfg.B):
        for s in range(n_sets):
            got = last["idx"][b, s, :int(last["cnt"][b, s])]
            assert np.array_equal(got, ref32[b][s]), (b, s)
            common = np.intersect1d(got, ref64[b][s]).size
            assert common >= 0.99 * ref64[b][s].size
    o_d, _ = oa.sparse_attn(last["qd"], last["k_before"], kv.v, kv.block_table, cfg.page_size, mode,
                            last["idx"], last["cnt"], kv.prefix_len,
                            np.full(cfg.B, last["tail_len"], dtype=np.int32), scale)
    assert float(np.max(np.abs(last["dout"] - o_d))) <= 1e-2
