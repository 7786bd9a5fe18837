"""bench.py's command-line contract on a machine without a GPU (CPU only): more
than one GPU is refused with a message, and the JSON line is only printed by a
real run; and the warm-up's stopping rule (steady_chunks) on simulated call
times: steady, rising, jittering, and a steady slow spell before a step."""

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


def _bench_module():
    import importlib.util

    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


class _Device:
    """A stand-in for back-to-back calls: per-call time from a function of the time spent."""

    def __init__(self, per_call_ms):
        self.per_call_ms = per_call_ms
        self.spent = 0.0
        self.chunks = []

    def __call__(self, n):
        ms = n * self.per_call_ms(self.spent)
        self.spent += ms
        self.chunks.append(n)
        return ms


def test_warmup_stops_at_the_floor_when_steady():
    b = _bench_module()
    dev = _Device(lambda t: 0.01)
    spent = b.steady_chunks(dev, min_ms=50.0, max_ms=1000.0)
    assert 50.0 <= spent < 50.0 + 2 * b.WARMUP_CHUNK_MS + 1e-9
    assert dev.chunks[0] == 10 and all(n == dev.chunks[1] for n in dev.chunks[1:])
    assert abs(dev.chunks[1] * 0.01 - b.WARMUP_CHUNK_MS) < 0.011  # chunks of about 20 ms


def test_warmup_waits_while_the_call_time_moves():
    b = _bench_module()
    # clocks rising: 5 % faster per 20 ms until 200 ms, flat from then on
    dev = _Device(lambda t: 0.01 * 0.95 ** (min(t, 200.0) / 20.0))
    spent = b.steady_chunks(dev, min_ms=50.0, max_ms=1000.0)
    assert 200.0 < spent < 200.0 + 3 * b.WARMUP_CHUNK_MS


def test_a_steady_slow_spell_is_covered_only_by_the_floor():
    """Low clocks that hold steady, then a step: the chunk-to-chunk test stops inside the slow
    spell, so only the floor (the headline's 1 s) gets past a step that comes before it."""
    b = _bench_module()
    slow_then_fast = lambda t: 0.012 if t < 400.0 else 0.01
    assert b.steady_chunks(_Device(slow_then_fast), min_ms=50.0, max_ms=1000.0) < 400.0
    assert b.steady_chunks(_Device(slow_then_fast), min_ms=b.STEP_WARMUP_MIN_MS,
                           max_ms=b.STEP_WARMUP_MAX_MS) >= b.STEP_WARMUP_MIN_MS


def test_warmup_is_bounded():
    b = _bench_module()
    k = {"i": 0}

    def jitter(t):  # never two chunks within 1 %
        k["i"] += 1
        return 0.01 if k["i"] % 2 else 0.0105

    dev = _Device(jitter)
    spent = b.steady_chunks(dev, min_ms=50.0, max_ms=300.0)
    assert 300.0 <= spent < 300.0 + 2 * b.WARMUP_CHUNK_MS


def test_warmup_floor_outlasts_a_slow_ramp():
    """A ramp too slow for the chunk-to-chunk test still gets the whole floor."""
    b = _bench_module()
    dev = _Device(lambda t: 0.012 - 0.002 * min(t, 1000.0) / 1000.0)
    spent = b.steady_chunks(dev, min_ms=b.STEP_WARMUP_MIN_MS, max_ms=b.STEP_WARMUP_MAX_MS)
    assert spent >= b.STEP_WARMUP_MIN_MS
