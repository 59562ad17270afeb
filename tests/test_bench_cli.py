"""bench.py's command-line contract, checked on the host (no GPU needed):
it measures one GPU and refuses more, before touching a device."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench(*args, env=None):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True, text=True,
                          timeout=120, env=env)


def test_more_than_one_gpu_is_refused():
    r = _bench("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_a_multi_rank_launch_is_refused():
    env = dict(os.environ, WORLD_SIZE="2", RANK="0", LOCAL_RANK="0")
    r = _bench(env=env)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_unknown_workload_is_an_argument_error():
    r = _bench("--config", "no_such_workload")
    assert r.returncode == 2
    assert "invalid choice" in r.stderr
