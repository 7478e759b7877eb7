"""bench.py's command line: one GPU only, refused before any GPU work; flags parsed (runs on the CPU)."""
import os
import subprocess
import sys

import pytest

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


def test_sweep_flag_is_parsed():
    import importlib.util
    spec = importlib.util.spec_from_file_location("bench_cli_probe", os.path.join(ROOT, "bench.py"))
    bench = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(bench)
    argv = sys.argv
    try:
        sys.argv = ["bench.py", "--sweep"]
        assert bench.parse().sweep
        sys.argv = ["bench.py"]
        assert not bench.parse().sweep
    finally:
        sys.argv = argv


def test_sweep_refuses_more_than_one_gpu_too():
    r = _run(["--sweep", "--gpus", "2"])
    assert r.returncode == 2 and r.stdout == ""


def test_kv_layout_flag_is_parsed():
    import importlib.util
    spec = importlib.util.spec_from_file_location("bench_cli_probe2", os.path.join(ROOT, "bench.py"))
    bench = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(bench)
    argv = sys.argv
    try:
        sys.argv = ["bench.py"]
        assert bench.parse().kv_layout == "token"
        sys.argv = ["bench.py", "--kv-layout", "head"]
        assert bench.parse().kv_layout == "head"
        sys.argv = ["bench.py", "--kv-layout", "diagonal"]
        with pytest.raises(SystemExit):
            bench.parse()
    finally:
        sys.argv = argv
