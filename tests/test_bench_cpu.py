"""bench.py's command-line contract on the CPU: more than one GPU is refused
with a message, and a run without a GPU fails loudly instead of falling back."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(*args, env=None):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], cwd=ROOT,
                          capture_output=True, text=True, timeout=300, env=env)


def test_more_than_one_gpu_is_refused():
    r = _run("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


def test_world_size_above_one_is_refused():
    env = dict(os.environ, WORLD_SIZE="4")
    r = _run(env=env)
    assert r.returncode == 2 and "one GPU" in r.stderr


def test_no_gpu_fails_loudly():
    import torch
    if torch.cuda.is_available():
        return                                    # only meaningful where there is no GPU
    r = _run("--steps", "1", "--warmup", "0", "--no-cpu-baseline")
    assert r.returncode == 2
    assert "needs a GPU" in r.stderr
    assert r.stdout.strip() == ""
