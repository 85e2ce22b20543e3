"""bench.py's measured HBM traffic: the committed rocprofv3 byte counts are
reported only for the device sources they were taken on."""
import json
import os

import bench
from quantized_delta_rule_decode_amd import build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _record():
    return json.load(open(os.path.join(ROOT, "profiles", "traffic.json")))


def test_traffic_reported_for_the_profiled_sources(monkeypatch):
    rec = _record()
    monkeypatch.setattr(build, "device_source_hash", lambda: rec["kernel_source_sha256_16"])
    for cid in (4, 5):
        entry = rec[f"config{cid}"]
        got = bench.measured_traffic(cid)
        assert got == entry["fetch_bytes_per_step"] + entry["write_bytes_per_step"]
        assert got > 0


def test_traffic_withheld_once_the_sources_change(monkeypatch):
    rec = _record()
    monkeypatch.setattr(build, "device_source_hash", lambda: "0" * 16 if rec["kernel_source_sha256_16"] != "0" * 16 else "1" * 16)
    assert bench.measured_traffic(4) is None
    assert bench.measured_traffic(5) is None


def test_traffic_withheld_for_an_unprofiled_workload(monkeypatch):
    rec = _record()
    monkeypatch.setattr(build, "device_source_hash", lambda: rec["kernel_source_sha256_16"])
    assert bench.measured_traffic(99) is None
