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
    cfg = synth.CONFIGS["stress_128k"].with_(L=2048, top_k=256)
    rec = bench.cpu_baseline(cfg, 0.5)
    assert rec["kind"] == "oracle" and rec["unit"] == "GB/s" and rec["value"] > 0 and rec["cores"] >= 1
    assert "replicated" in rec["sample"] and "one sequence x one KV head" in rec["sample"]
    json.dumps(rec)


def test_default_workload_is_the_largest_one_gpu_config():
    sys.path.insert(0, ROOT)
    import bench
    from long_context_self_amd import synth
    cfgs = [c for c in synth.CONFIGS.values() if c.mode in ("shared", "per_kv_head")]
    biggest = max(cfgs, key=lambda c: c.B * c.L * c.Hkv)
    assert bench.DEFAULT_CONFIG == biggest.name == "stress_128k"
