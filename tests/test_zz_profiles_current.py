"""The committed counter summary under profiles/ was taken on the kernel
sources as they stand (bench.py reports `roofline.traffic` only then).
Collected last so that a stale summary cannot hide other results."""
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_committed_traffic_matches_the_current_sources():
    sha = bench.kernel_source_sha()
    assert len(sha) == 16 and all(c in "0123456789abcdef" for c in sha)
    with open(bench.TRAFFIC_FILE) as fh:
        t = json.load(fh)
    assert t["kernel_source_sha"] == sha, "profiles/ counter summary taken on other kernel sources"
    assert abs(t["bytes_per_launch"] - (t["fetch_bytes"] + t["write_bytes"])) <= 1
