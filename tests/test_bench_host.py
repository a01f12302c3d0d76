"""Host-side checks of bench.py: the one-GPU rule and the counter-traffic
bookkeeping (no GPU needed)."""
import json
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_traffic_is_reported_only_for_the_measured_sources(tmp_path):
    for path in (bench.TRAFFIC_FILE, bench.C128_PREFILL_TRAFFIC, bench.C128_DECODE_TRAFFIC,
                 bench.RING_TRAFFIC):
        t = json.load(open(path))
        assert 0.99 < t["traffic_over_algorithmic"] < 1.1
        srcs = tuple(t.get("kernel_sources", bench.KERNEL_SOURCES))
        p = tmp_path / os.path.basename(path)
        # counters taken on the current sources are reported ...
        p.write_text(json.dumps(dict(t, kernel_sha=bench.kernel_source_sha(srcs))))
        assert bench.measured_traffic(str(p)) == t["bytes_per_launch"]
        # ... counters taken on other sources are not
        p.write_text(json.dumps(dict(t, kernel_sha="0" * 64)))
        assert bench.measured_traffic(str(p)) is None
    assert bench.measured_traffic(str(tmp_path / "missing.json")) is None


