"""CPU checks of bench.py's command-line contract that need no GPU: a run
asked for more than one GPU exits at once with a message (this build
measures one GPU), and every workload name parses."""
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    msg = json.loads(r.stdout.strip().splitlines()[-1])
    assert "one GPU" in msg["error"]


def test_workload_names_and_layer_defaults():
    sys.path.insert(0, ROOT)
    import bench
    for wl, layers in (("stagger128k", 64), ("long1m", 40), ("tiny", 64), ("lmhead_verify", 64)):
        sys.argv = ["bench.py", "--workload", wl]
        assert bench.parse().layers == layers
    sys.argv = ["bench.py", "--workload", "long1m", "--layers", "8"]
    assert bench.parse().layers == 8
