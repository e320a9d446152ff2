"""Host-side checks of bench.py (no GPU): the one-GPU contract and the
pieces of its report that do not need a device."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.parametrize("n", ["2", "8"])
def test_more_than_one_gpu_is_refused(n):
    """--gpus N > 1 exits (status 2) with one JSON line that says the
    benchmark runs on one GPU, before touching torch or the device."""
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", n], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 2
    msg = json.loads(r.stdout.strip().splitlines()[-1])
    assert "one GPU" in msg["error"]


def test_traffic_is_reported_only_for_the_measured_kernel():
    """roofline.traffic comes from the committed counter record only while
    the headline kernel's sources hash as they did when it was taken;
    otherwise it is null."""
    sys.path.insert(0, ROOT)
    import bench
    h = bench._kernel_source_hash()
    assert isinstance(h, str) and len(h) == 16
    rec = json.load(open(os.path.join(ROOT, "profiles", "qgemv_layer_8b_m1_one_launch_traffic.json")))
    want = rec["traffic_bytes_per_launch"] if rec["kernel_source_hash"] == h else None
    assert bench._profile_traffic(h) == want
    assert bench._profile_traffic("0" * 16) is None
