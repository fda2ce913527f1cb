"""The benchmark's command-line contract (CPU only: nothing here touches a GPU)."""
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    """bench.py measures one GPU: --gpus N > 1 exits with a message, before
    importing anything that would look for a device."""
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=60)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


def test_stored_counter_summaries_parse():
    """Every committed HBM-traffic summary carries a record the benchmark can
    read: per-launch bytes, the calibration factors and a source hash."""
    prof = os.path.join(ROOT, "profiles")
    found = 0
    for name in sorted(os.listdir(prof)):
        if not name.endswith("_hbm_traffic.md"):
            continue
        with open(os.path.join(prof, name)) as fh:
            recs = [l for l in fh if l.startswith("<!-- traffic-json: ")]
        assert len(recs) == 1, name
        rec = json.loads(recs[0][len("<!-- traffic-json: "):].rsplit(" -->", 1)[0])
        assert rec["bytes_per_launch"] > 0 and rec["algorithmic_bytes_per_launch"] > 0, name
        assert 0.4 < rec["calibration"]["fetch_factor"] < 4.0, name
        assert len(rec["src_hash"]) == 16, name
        found += 1
    assert found >= 10


def test_mid_workload_takes_the_mid_size_gemm():
    """Every call of the benchmark's `mid` workload is a shape the mid-size
    GEMM takes (by the rule restated in the tests), so the workload measures
    that kernel; none of the decode workload's calls is."""
    sys.path.insert(0, ROOT)
    import bench
    from tests.gpu_helpers import mid_rule
    mid, _ = bench.workload_configs("mid")
    assert len(mid) == 4 and all(mid_rule(m, n, k) > 0 for (m, k, n) in mid)
    decode, _ = bench.workload_configs("decode")
    assert all(mid_rule(m, n, k) == 0 for (m, k, n) in decode)

