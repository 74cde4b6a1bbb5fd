"""bench.py's command-line contract on the host: more than one GPU is
refused with a message and exit status 2 before anything touches a GPU."""

import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout == ""


def test_stored_traffic_belongs_to_its_workload():
    """The committed HBM counter figures are reported only for the workload
    and kernel sources they were taken on."""
    sys.path.insert(0, ROOT)
    import json

    import bench
    from rejection_sampling_verifier_amd import workloads as W

    with open(bench.TRAFFIC_FILE) as f:
        t = json.load(f)
    assert t["workload"] == W.CONFIGS[2].name
    for c, w in W.CONFIGS.items():
        got = bench.stored_traffic(w.name)
        if c != 2:
            assert got is None, w.name
        elif t["kernel_source_sha"] == bench.kernel_source_sha():
            assert got == t["hbm_bytes_per_launch"]
        else:
            assert got is None
