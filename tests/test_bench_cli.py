"""bench.py's command line on the host: it refuses more than one GPU, and
without a GPU it fails instead of printing a result line (there is no CPU
path to fall back to)."""

import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                          capture_output=True, text=True, timeout=300, cwd=ROOT)


def test_more_than_one_gpu_is_refused():
    r = _run("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU only" in r.stdout + r.stderr
    assert not any(line.startswith("{") for line in r.stdout.splitlines())


def test_no_result_line_without_a_gpu():
    import torch
    if torch.cuda.is_available():
        return
    r = _run("--steps", "1", "--warmup", "1", "--no-cpu", "--no-extra")
    assert r.returncode != 0
    assert not any(line.startswith("{") for line in r.stdout.splitlines())
