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


def test_every_kernel_leg_names_its_kernel():
    # each single-kernel workload reports the entry point and kernels it times
    import argparse
    sys.path.insert(0, ROOT)
    import bench
    captured = {}
    orig = argparse.ArgumentParser.parse_args

    def grab(self, *a, **k):
        for act in self._actions:
            if act.dest == "workload":
                captured["choices"] = list(act.choices)
        return orig(self, *a, **k)
    sys.argv = ["bench.py"]
    argparse.ArgumentParser.parse_args = grab
    try:
        bench.parse()
    finally:
        argparse.ArgumentParser.parse_args = orig
    rounds = {"stagger128k", "long1m", "remote1m", "tiny"}
    legs = [w for w in captured["choices"] if w not in rounds]
    assert legs and all(w in bench.KERNEL_OF for w in legs), set(legs) - set(bench.KERNEL_OF)
