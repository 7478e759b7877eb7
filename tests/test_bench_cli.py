"""bench.py's command line: one GPU only, refused before any GPU work (runs on the CPU)."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(args, env_extra=None):
    env = dict(os.environ)
    env.update(env_extra or {})
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], cwd=ROOT, env=env,
                          capture_output=True, text=True, timeout=60)


def test_more_than_one_gpu_is_refused_with_a_message():
    r = _run(["--gpus", "2"])
    assert r.returncode == 2
    assert "exactly one GPU" in r.stderr
    assert r.stdout == ""  # no JSON line


def test_multi_rank_launch_is_refused():
    r = _run([], {"WORLD_SIZE": "8"})
    assert r.returncode == 2
    assert "exactly one GPU" in r.stderr
