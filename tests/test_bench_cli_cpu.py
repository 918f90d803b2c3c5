"""bench.py's command line on the host: more than one GPU is refused before any
GPU work (one MI355X per box; the token-parallel sharding needs no collective
and is not exercised)."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(args, env_extra=None):
    env = dict(os.environ)
    env.update(env_extra or {})
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], cwd=ROOT,
                          env=env, capture_output=True, text=True, timeout=120)


def test_more_than_one_gpu_is_refused():
    r = _run(["--gpus", "2", "--steps", "1", "--warmup", "1"])
    assert r.returncode == 2, (r.returncode, r.stderr[-500:])
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""  # no JSON line


def test_a_multi_rank_launch_is_refused():
    r = _run(["--gpus", "1"], {"WORLD_SIZE": "8", "RANK": "0", "LOCAL_RANK": "0"})
    assert r.returncode == 2, (r.returncode, r.stderr[-500:])
    assert r.stdout.strip() == ""
