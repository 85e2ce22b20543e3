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


def test_traffic_of_the_dominant_launch(monkeypatch):
    from quantized_delta_rule_decode_amd import synth
    rec = _record()
    monkeypatch.setattr(build, "device_source_hash", lambda: rec["kernel_source_sha256_16"])
    for cid in (4, 5):
        cfg = synth.CONFIGS[cid]
        kernel = bench.dominant_kernel(cfg)
        entry = rec[f"config{cid}"]
        assert kernel == entry["dominant_kernel"] and kernel in entry["kernel_bytes"]
        got = bench.measured_traffic(cid, kernel)
        assert got == entry["kernel_bytes"][kernel]["fetch"] + entry["kernel_bytes"][kernel]["write"]
        assert 0 < got <= bench.measured_traffic(cid)
        # measured bytes of the launch within a few percent of its algorithmic bytes
        kbytes = bench.algorithmic_bytes(cfg, synth.static_tables(cfg), integer_heads_only=True)
        assert 1.0 <= got / kbytes < 1.06
    assert bench.measured_traffic(4, "void qdr::no_such_kernel(qdr::LaunchArgs)") is None


def test_traffic_withheld_once_the_sources_change(monkeypatch):
    rec = _record()
    monkeypatch.setattr(build, "device_source_hash", lambda: "0" * 16 if rec["kernel_source_sha256_16"] != "0" * 16 else "1" * 16)
    assert bench.measured_traffic(4) is None
    assert bench.measured_traffic(5) is None


def test_traffic_withheld_for_an_unprofiled_workload(monkeypatch):
    rec = _record()
    monkeypatch.setattr(build, "device_source_hash", lambda: rec["kernel_source_sha256_16"])
    assert bench.measured_traffic(99) is None


def test_algorithmic_bytes_of_the_gdn_pool():
    """The benchmark pool's bytes per step, written out from its head counts
    and the per-head sizes of each kind: 128 x 128 codes of b bits (FP16
    pivots 32 KiB), fp32 r and c (1 KiB) for integer heads, each read and
    written once, plus q, k, v, beta, the scalar gate and o per head-step."""
    from quantized_delta_rule_decode_amd import synth
    cfg = synth.CONFIGS[4]
    counts = {16: 46, 8: 691, 6: 991, 4: 576}
    codes = sum(n * 128 * 128 * b // 8 for b, n in counts.items())
    scales = sum(n for b, n in counts.items() if b <= 8) * 2 * 128 * 4
    vectors = cfg.H * (3 * 128 * 4 + 4 + 4 + 128 * 4)
    per_request = 2 * (codes + scales) + vectors
    assert per_request * cfg.B == 35_231_105_024
    t = synth.static_tables(cfg)
    assert bench.algorithmic_bytes(cfg, t) == per_request * cfg.B
    # the integer launch's share: the FP16 pivot heads are another launch
    fp16 = counts[16] * (2 * 128 * 128 * 2 + 3 * 128 * 4 + 4 + 4 + 128 * 4)
    assert bench.algorithmic_bytes(cfg, t, integer_heads_only=True) == (per_request - fp16) * cfg.B
