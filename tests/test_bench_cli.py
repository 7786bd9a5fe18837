"""bench.py's command-line contract on a machine without a GPU (CPU only): more
than one GPU is refused with a message, and the JSON line is only printed by a
real run."""

from __future__ import annotations

import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], cwd=ROOT,
                          stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True, timeout=300)


def test_more_than_one_gpu_is_refused():
    p = run("--gpus", "2", "--steps", "1", "--warmup", "0")
    assert p.returncode == 2
    assert "one GPU" in p.stderr
    assert p.stdout.strip() == ""


def test_help_lists_the_contract_flags():
    p = run("--help")
    assert p.returncode == 0
    for flag in ("--gpus", "--steps", "--warmup"):
        assert flag in p.stdout
