"""Host logic of bench.py that needs no GPU: the counter-derived traffic is
reported only for the top-K source and workload the counters were taken on."""
import hashlib
import json

import bench


def test_measured_traffic_requires_matching_source_and_workload(tmp_path, monkeypatch):
    src, hdr = tmp_path / "topk.hip", tmp_path / "device_common.h"
    src.write_bytes(b"kernel source v1")
    hdr.write_bytes(b"helpers v1")
    sha = hashlib.sha256(b"kernel source v1helpers v1").hexdigest()
    rec = tmp_path / "topk_traffic.json"
    rec.write_text(json.dumps({"source_sha256": sha, "workload": "w", "fetch_bytes_per_launch": 1000,
                               "write_bytes_per_launch": 24}))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(rec))
    monkeypatch.setattr(bench, "TOPK_SOURCES", (str(src), str(hdr)))
    assert bench.measured_traffic("w") == 1024
    assert bench.measured_traffic("other") is None
    hdr.write_bytes(b"helpers v2")                        # an inlined helper changed since the counters
    assert bench.measured_traffic("w") is None
    hdr.write_bytes(b"helpers v1")
    assert bench.measured_traffic("w") == 1024
    src.write_bytes(b"kernel source v2")                  # the kernel changed since the counters
    assert bench.measured_traffic("w") is None
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "missing.json"))
    assert bench.measured_traffic("w") is None

