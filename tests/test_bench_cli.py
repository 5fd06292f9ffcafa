"""Host-side checks of bench.py's command line and of what it reads (no GPU).

bench.py measures one GPU: any other --gpus value must end the run with a
non-zero status and a message, before anything touches a device.  The
profile it takes the HBM traffic figure from must name the kernel sources it
was measured on, and the figure is used only while they are unchanged.
"""

import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)


@pytest.mark.parametrize("n", ["2", "8", "0"])
def test_more_than_one_gpu_is_refused(n):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", n],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in (r.stdout + r.stderr)


def test_traffic_profile_matches_its_sources():
    import bench

    path = os.path.join(ROOT, "profiles", "traffic_headline_causal_bf16.json")
    rec = json.load(open(path))
    for name in bench.KERNEL_SOURCES:
        assert os.path.exists(os.path.join(ROOT, "online_softmax_streaming_amd", "csrc", name)), name
    got = bench.traffic_from_profiles("headline_causal_bf16")
    if rec.get("source_hash") == bench.source_hash():
        assert got == rec["hbm_bytes_per_launch"] and got > 0
    else:
        assert got is None  # stale counters are not reported
    assert bench.traffic_from_profiles("decode_bf16") is None
