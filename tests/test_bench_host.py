"""Host-side checks of bench.py's measured-traffic record (no GPU).

The bench line reports the AnnSA kernel's HBM traffic from a counter record
kept under profiles/, keyed by the SHA-256 of the kernel's sources.  These
tests check that the record is well formed, that the files it is keyed on
exist, and that a record whose key or workload does not match is refused.
"""
import json
import os

from tests.conftest import ROOT

import bench


def test_traffic_record_is_well_formed():
    with open(bench.TRAFFIC_FILE) as f:
        rec = json.load(f)
    assert rec["kernel"] == bench.ANNSA_KERNEL
    assert rec["traffic_bytes"] > 0
    assert rec["fetch_scale"] > 0 and rec["write_scale"] > 0
    scaled = (rec["fetch_scale"] * rec["fetch_kib_per_dispatch"]
              + rec["write_scale"] * rec["write_kib_per_dispatch"]) * 1024
    assert abs(scaled - rec["traffic_bytes"]) <= 1e-6 * scaled
    assert rec["sources"] == bench.KERNEL_SOURCES
    for rel in rec["sources"]:
        assert os.path.isfile(os.path.join(ROOT, rel)), rel


def test_stale_or_foreign_records_are_refused(tmp_path, monkeypatch):
    with open(bench.TRAFFIC_FILE) as f:
        rec = json.load(f)
    rec["sources_sha256"] = "0" * 64
    path = tmp_path / "rec.json"
    path.write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(path))
    assert bench.measured_traffic(rec["config"], rec["out_dtype"])[0] is None
    rec["sources_sha256"] = bench.kernel_sources_sha256()
    path.write_text(json.dumps(rec))
    assert bench.measured_traffic(rec["config"], rec["out_dtype"])[0] == rec["traffic_bytes"]
    assert bench.measured_traffic("tiny", rec["out_dtype"])[0] is None
    assert bench.measured_traffic(rec["config"], "bf16")[0] is None
