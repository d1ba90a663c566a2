"""bench.py's command-line contract on the CPU: it measures one GPU only and
refuses more, before touching a GPU."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def run_bench(args, extra_env=None):
    env = dict(os.environ)
    env.update(extra_env or {})
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py")] + args, cwd=ROOT, env=env,
                          stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True, timeout=120)


def test_more_than_one_gpu_is_refused():
    p = run_bench(["--gpus", "2"])
    assert p.returncode == 2
    assert "one GPU" in p.stderr
    assert p.stdout == ""


def test_world_size_above_one_is_refused():
    p = run_bench([], {"WORLD_SIZE": "2"})
    assert p.returncode == 2
    assert "one GPU" in p.stderr
