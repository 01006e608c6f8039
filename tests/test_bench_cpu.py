"""Host-side behaviour of bench.py (no GPU): the one-GPU contract and argument checks
exit before any device work, and the clock-settle phase can be switched off."""

import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)


def _run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                          capture_output=True, text=True, timeout=120)


def test_more_than_one_gpu_is_refused():
    r = _run("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_world_size_above_one_is_refused():
    env = dict(os.environ, WORLD_SIZE="4")
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py")], capture_output=True,
                       text=True, timeout=120, env=env)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_bad_step_counts_are_refused():
    assert _run("--steps", "0").returncode == 2
    assert _run("--warmup", "-1").returncode == 2


def test_clock_settle_off():
    import bench
    calls = []
    assert bench.clock_settle(lambda: calls.append(1), 0.0, 4) is None
    assert bench.clock_settle(lambda: calls.append(1), -5.0, 4) is None
    assert calls == []


def test_gelu_in_two_layers_is_refused():
    r = _run("--workload", "chain", "--fuse-gelu", "--gelu-down")
    assert r.returncode == 2
    assert "pick one" in r.stderr
