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
