"""CPU checks of bench.py's bookkeeping: the kernels whose HBM traffic its
roofline objects report are named as the committed profile names them, and
a request for more than one GPU exits with a message."""
import json
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_roofline_kernels_are_in_the_traffic_profile():
    with open(os.path.join(ROOT, "profiles", "traffic_prefill128k_decode128k.json")) as fh:
        names = set(json.load(fh)["kernels"])
    assert bench.PREFILL_KERNEL in names
    for k in bench.DECODE_KERNELS:
        assert k in names
    # exact names: a prefix of another kernel's name would add its bytes
    for k in (bench.PREFILL_KERNEL, *bench.DECODE_KERNELS):
        assert [n for n in names if n.startswith(k)] == [k]


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode != 0
    assert "single GPU" in r.stderr
