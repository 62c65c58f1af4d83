"""Host-side checks of bench.py (no GPU): the one-GPU contract and the
recorded-traffic lookup."""
import os
import re
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], cwd=ROOT,
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout == ""


def test_recorded_traffic_follows_the_gemm_source_hash_and_workload():
    h = bench.gemm_source_hash()
    assert re.fullmatch(r"[0-9a-f]{64}", h)
    text = open(bench.TRAFFIC_PROFILE).read()
    m = re.search(r"^source_sha256:\s*([0-9a-f]{64})\s*$", text, re.M)
    assert m, "the traffic profile records the hash of the sources it was taken on"
    w = re.search(r"^workload:\s*(\S+)\s*$", text, re.M)
    assert w, "the traffic profile names the workload it was taken on"
    t = bench.recorded_traffic(w.group(1))
    if m.group(1) == h:
        assert t is not None and t > 0
    else:
        assert t is None   # counters taken on other sources are not reported
    # another workload never reports these counters as its own
    assert bench.recorded_traffic("inkling_default_h6144") is None
    assert bench.recorded_traffic("decode_h6144") is None
