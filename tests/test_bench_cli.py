"""bench.py's command-line contract on the host (no GPU needed): one GPU only, and the
oracle's CPU baseline leg runs without touching a device."""
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in r.stderr and r.stdout.strip() == ""


def test_cpu_baseline_leg_on_a_bounded_sample():
    """The oracle leg alone: a bounded sample of the 32K workload timed on the host cores."""
    sys.path.insert(0, ROOT)
    import bench
    from long_context_self_amd import synth
    cfg = synth.CONFIGS["llama8b_32k"].with_(L=2048, top_k=256)
    kv = synth.make_paged_kv(cfg, seed=0)
    q = synth.make_queries(cfg, kv, cfg.n_q, seed=0)
    qd = [synth.make_queries(cfg, kv, 1, seed=0, tag=100 + j) for j in range(cfg.n_draft)]
    rec = bench.cpu_baseline(cfg, kv, q, qd, None, 0.5)
    assert rec["kind"] == "oracle" and rec["unit"] == "GB/s" and rec["value"] > 0 and rec["cores"] >= 1
    json.dumps(rec)
