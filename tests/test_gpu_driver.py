"""The speculative-iteration driver runs verify -> select -> k draft steps with drift
through the library, and the selection keeps finding the planted critical keys."""
import math

import pytest

from long_context_self_amd import synth

from gpu_helpers import require_gpu

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("mode", ["shared", "per_kv_head"])
def test_driver_loop_with_drift(mode):
    require_gpu()
    from long_context_self_amd import driver
    cfg = synth.CONFIGS["llama8b_32k"].with_(L=8192, top_k=512, crit_frac=0.01, mode=mode)
    res = driver.run(cfg, iters=6, drift=0.1, seed=1)
    med = res["median"]
    for key in ("verify_us", "select_us", "draft_us", "iter_us"):
        assert math.isfinite(med[key]) and med[key] > 0
    assert med["moved_rows"] > 0
    # a set chosen blindly would hold budget / L of the critical keys; the logit-guided
    # set must do clearly better, before and after the keys drift
    blind = (cfg.n_sink + cfg.top_k + cfg.n_recent) / cfg.L
    print(f"{mode}: recall first {res['recall_first']:.3f} last {res['recall_last']:.3f} (blind {blind:.3f})")
    assert res["recall_first"] > 2 * blind and res["recall_last"] > 2 * blind
