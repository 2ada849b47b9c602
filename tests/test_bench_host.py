"""Host-side checks of bench.py (no GPU): it refuses more than one GPU before
touching one, and the committed scan traffic records are current for the scan
sources (so the headline roofline's `traffic` is reported, not null) and hold
at least the algorithmic bytes of a launch."""
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


def test_scan_traffic_records_are_current():
    import bench
    for workload in ("m2p7b_stack", "m130m_layer"):
        with open(os.path.join(ROOT, "profiles", f"scan_{workload}_traffic.json")) as f:
            rec = json.load(f)
        assert rec["scan_source_sha256_16"] == bench.scan_source_hash(), (
            f"{workload}: the scan sources changed since its counters were taken")
        got = bench.load_traffic(workload, 1)
        assert got == rec["hbm_bytes_per_launch"]
        assert got >= rec["algorithmic_bytes_per_launch"]
        # the calibration of the fetch counter against a 256 MiB copy
        assert abs(rec["fetch_scale"] * rec["copy_fetch_size_kib_raw"] - 262144) < 16
