"""The rocprofv3 summary tool's traffic scaling (CPU): counters are scaled by what the
same counter reads for the calibration copy, which is the last large copy dispatch."""
import json
import sqlite3

from long_context_self_amd import profile_summary as ps


def _db(path, counter, rows):
    c = sqlite3.connect(path)
    c.execute("create table counters_collection (dispatch_id integer, kernel_name text, counter_name text, "
              "value real)")
    c.executemany("insert into counters_collection values (?, ?, ?, ?)",
                  [(i, name, counter, v) for i, (name, v) in enumerate(rows)])
    c.commit()
    c.close()


def test_calibration_is_the_last_large_copy(tmp_path):
    GiB_kib = 1 << 20
    copy = ps.COPY_KERNEL
    k = "void lcs::(anonymous namespace)::attn_kernel<128, 3, 0, false>(lcs::AttnArgs)"
    # two 2 GiB KV replicas, a tiny copy, the 1 GiB calibration copy, a tiny copy, then the kernel;
    # FETCH_SIZE reads half of a copy's bytes, WRITE_SIZE all of them
    fetch = [(copy, GiB_kib), (copy, GiB_kib), (copy, 2.0), (copy, GiB_kib / 2), (copy, 2.0), (k, 3000.0)]
    write = [(copy, 2 * GiB_kib), (copy, 2 * GiB_kib), (copy, 0.0), (copy, GiB_kib), (copy, 0.0), (k, 500.0)]
    fdb, wdb = str(tmp_path / "f.db"), str(tmp_path / "w.db")
    _db(fdb, "FETCH_SIZE", fetch)
    _db(wdb, "WRITE_SIZE", write)
    out = tmp_path / "t.json"
    ps.main(["traffic", "--fetch", fdb, "--write", wdb, "--copy-bytes", str(1 << 30),
             "--kernel", "attn_kernel<128, 3, 0, false>", "--algorithmic-bytes", str(7000 * 1024),
             "--command-fetch", "f", "--command-write", "w", "--out", str(out)])
    rec = json.load(open(out))
    assert rec["FETCH_SIZE_factor"] == 2.0 and rec["WRITE_SIZE_factor"] == 1.0
    assert rec["hbm_bytes_per_launch"] == (2 * 3000 + 500) * 1024


def test_per_call_traffic_is_the_median_dispatch(tmp_path):
    """A kernel whose first call takes a longer one-time path (here three times the bytes)
    is charged its steady per-call traffic, not the mean that the first call pulls up."""
    copy = ps.COPY_KERNEL
    k = "void lcs::(anonymous namespace)::collect_kernel<0>(lcs::SelArgs)"
    fetch = [(copy, 1024.0), (k, 300.0), (k, 100.0), (k, 100.0), (k, 100.0), (k, 100.0)]
    write = [(copy, 1024.0), (k, 30.0), (k, 10.0), (k, 10.0), (k, 10.0), (k, 10.0)]
    fdb, wdb = str(tmp_path / "f.db"), str(tmp_path / "w.db")
    _db(fdb, "FETCH_SIZE", fetch)
    _db(wdb, "WRITE_SIZE", write)
    out = tmp_path / "t.json"
    ps.main(["traffic", "--fetch", fdb, "--write", wdb, "--copy-bytes", str(1 << 20),
             "--kernel", "collect_kernel<0>", "--algorithmic-bytes", str(110 * 1024),
             "--command-fetch", "f", "--command-write", "w", "--out", str(out)])
    rec = json.load(open(out))
    ent = rec["kernels"]["collect_kernel<0>"]
    assert ent["FETCH_SIZE_kib_median"] == 100.0 and ent["FETCH_SIZE_kib_max"] == 300.0
    assert ent["FETCH_SIZE_kib_mean"] == 140.0
    assert rec["hbm_bytes_per_launch"] == 110 * 1024
    assert rec["traffic_over_algorithmic"] == 1.0
