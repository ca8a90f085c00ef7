"""Host-side checks of bench.py (no GPU): the one-GPU contract and the rule
that the measured HBM traffic is reported only while the kernel sources it
was taken from are unchanged."""

import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_traffic_reported_only_for_the_profiled_sources(tmp_path, monkeypatch):
    f = tmp_path / "traffic.json"
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(f))
    assert bench.measured_traffic(1) is None  # no file
    f.write_text(json.dumps({"kernel_source_hash": bench.kernel_source_hash(), "traffic_bytes_per_launch": 123}))
    assert bench.measured_traffic(1) == 123
    f.write_text(json.dumps({"kernel_source_hash": "0" * 16, "traffic_bytes_per_launch": 123}))
    assert bench.measured_traffic(1) is None  # sources changed since the counters were taken
    f.write_text("not json")
    assert bench.measured_traffic(1) is None


def test_source_hash_covers_the_headline_kernel_files():
    for name in bench.HEADLINE_SOURCES:
        assert os.path.exists(os.path.join(bench.CSRC, name)), name
    assert "tah_encode.hip" in bench.HEADLINE_SOURCES and "tah_device.hpp" in bench.HEADLINE_SOURCES


def test_committed_traffic_file_names_its_commands():
    t = json.load(open(os.path.join(ROOT, "profiles", "k_encode_c5_roundtrip_traffic.json")))
    assert t["kernel"].startswith("void tah::k_encode<64")
    for cmd in t["commands"]["kernel"] + t["commands"]["copy"]:
        assert "rocprofv3 --pmc" in cmd and "bench.py" in cmd
    assert abs(t["traffic_bytes_per_launch"] - t["fetch_bytes_per_launch"] - t["write_bytes_per_launch"]) <= 1


def test_valu_figures_follow_the_same_staleness_rule(tmp_path, monkeypatch):
    f = tmp_path / "traffic.json"
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(f))
    sq = {"valu_lane_ops_per_element": 32.5, "valu_busy_frac": 0.8}
    f.write_text(json.dumps({"kernel_source_hash": bench.kernel_source_hash(), "sq": sq}))
    assert bench.measured_valu() == {"lane_ops_per_element": 32.5, "busy_frac": 0.8}
    f.write_text(json.dumps({"kernel_source_hash": "0" * 16, "sq": sq}))
    assert bench.measured_valu() is None
