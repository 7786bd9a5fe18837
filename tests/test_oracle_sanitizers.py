"""The CPU oracle under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

``oracle_sanitize_main.c`` drives every oracle entry point on small ragged
problems (tails, one-element rows, every lane count from 16 to 1024, empty
problems) and checks the closed forms it can state exactly.  It is compiled
together with ``oracle/adaln_oracle.c`` by gcc with both sanitizers and no
recovery, so an out-of-bounds access, a leak, signed overflow or any other
undefined behaviour in the oracle fails the run.  A copy of the oracle with
one planted off-by-one (a lane reading one vector past the end of its row)
must fail it, which shows the sanitizers are live in this build.
"""

from __future__ import annotations

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ORACLE = os.path.join(ROOT, "oracle", "adaln_oracle.c")
DRIVER = os.path.join(ROOT, "tests", "oracle_sanitize_main.c")
FLAGS = ["-std=c11", "-O1", "-g", "-fno-omit-frame-pointer", "-ffp-contract=off", "-fno-fast-math",
         "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fopenmp"]


def _build(src: str, out: str) -> None:
    r = subprocess.run(["gcc", *FLAGS, "-o", out, src, DRIVER, "-lm"], stdout=subprocess.PIPE,
                       stderr=subprocess.STDOUT, text=True)
    if r.returncode != 0 and "sanitizer" in r.stdout.lower() and "not" in r.stdout.lower():
        pytest.skip("gcc here has no sanitizer runtime: %s" % r.stdout[:200])
    assert r.returncode == 0, r.stdout


def _run(exe: str):
    env = dict(os.environ, OMP_NUM_THREADS="2", ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    return subprocess.run([exe], stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, env=env,
                          timeout=300)


@pytest.fixture(scope="module")
def gcc():
    if shutil.which("gcc") is None:
        pytest.skip("gcc not found")
    return "gcc"


def test_oracle_clean_under_asan_ubsan(gcc, tmp_path):
    exe = str(tmp_path / "orc_san")
    _build(ORACLE, exe)
    r = _run(exe)
    assert r.returncode == 0 and r.stdout.strip().endswith("ok"), r.stdout[-4000:]


def test_planted_overrun_is_caught(gcc, tmp_path):
    src = open(ORACLE).read()
    good = "for (int64_t v = l; v < nvec; v += L)\n      for (int e = 0; e < V; ++e) welford_push"
    assert good in src
    bad = src.replace(good, "for (int64_t v = l; v <= nvec; v += L)\n      for (int e = 0; e < V; ++e) welford_push")
    mutant = tmp_path / "adaln_oracle_overrun.c"
    mutant.write_text(bad)
    exe = str(tmp_path / "orc_san_mutant")
    _build(str(mutant), exe)
    r = _run(exe)
    assert r.returncode != 0 and "AddressSanitizer" in r.stdout, r.stdout[-2000:]
