"""Host-side checks of the benchmark's bookkeeping (no GPU)."""

import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_traffic_record_is_reported_only_for_its_workload():
    """The committed counter record belongs to one workload and one kernel source: other
    workloads get no traffic figure, and the record's own workload gets it only while the kernel
    source still has the digest the counters were taken on."""
    assert bench.measured_traffic("wan480p") == (None, None)
    assert bench.measured_traffic("stress") == (None, None)
    traffic, l2 = bench.measured_traffic(bench.TRAFFIC_WORKLOAD)
    import json
    rec = json.load(open(bench.TRAFFIC_FILE))
    if rec["source_sha256"] == bench.attn_source_digest():
        assert traffic == rec["bytes_per_launch"] and l2 == rec["l2_hit_rate"]
    else:
        assert (traffic, l2) == (None, None)
