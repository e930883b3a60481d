"""Host-side logic of bench.py (CPU): the one-GPU guard and the committed
counter records the bench line reads."""
import json
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_exits_before_any_gpu_work():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True, timeout=120)
    assert res.returncode == 2
    assert "one GPU" in res.stderr
    assert res.stdout == ""          # no JSON line for a run that did not happen


def test_traffic_record_follows_the_kernel_source(tmp_path, monkeypatch):
    """A counter record is used only while the kernel source it was taken
    from is unchanged."""
    prof = tmp_path / "profiles"
    prof.mkdir()
    rec = {"kernel_sha": bench.kernel_source_sha(), "bytes_per_launch": 123.0}
    (prof / "partition_demo_traffic.json").write_text(json.dumps(rec))
    sha = rec["kernel_sha"]
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "kernel_source_sha", lambda: sha)
    got = bench.load_traffic("demo")
    assert got is not None and got[0] == 123.0 and got[2] == rec["kernel_sha"]
    rec["kernel_sha"] = "0" * 16
    (prof / "partition_demo_traffic.json").write_text(json.dumps(rec))
    assert bench.load_traffic("demo") is None
    assert bench.load_traffic("absent") is None


def test_committed_traffic_records_are_consistent():
    """Each committed record: traffic = calibrated fetch + write bytes, the
    factors as measured against the probe copy, and the counters in KiB per
    dispatch times their factors."""
    prof = os.path.join(ROOT, "profiles")
    names = [f for f in os.listdir(prof) if f.startswith("partition_") and f.endswith("_traffic.json")]
    assert names
    for f in names:
        with open(os.path.join(prof, f)) as fh:
            r = json.load(fh)
        assert abs(r["fetch_bytes"] + r["write_bytes"] - r["bytes_per_launch"]) <= 1e-6 * r["bytes_per_launch"], f
        assert abs(r["counters_kib"]["FETCH_SIZE"] * 1024 * r["fetch_factor"] - r["fetch_bytes"]) <= 1e-6 * r["fetch_bytes"], f
        assert abs(r["counters_kib"]["WRITE_SIZE"] * 1024 * r["write_factor"] - r["write_bytes"]) <= 1e-6 * max(r["write_bytes"], 1.0), f
        # streaming launches (100 MB and more): traffic within a few percent
        # of the algorithmic bytes, i.e. no re-reads.  The tiny workload's
        # whole launch is 148 KB, of which the factor block that each
        # partition's workgroup reads again for its head is a large share.
        if r["algorithmic_bytes"] >= 100e6:
            assert 0.98 <= r["bytes_per_launch"] / r["algorithmic_bytes"] <= 1.05, f
