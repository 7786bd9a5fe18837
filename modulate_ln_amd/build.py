"""Build ``libadaln.so`` (HIP kernels for gfx950 + the C ABI) in-tree.

    python -m modulate_ln_amd.build

Every HIP source is compiled with hipcc for gfx950 only, with
``-ffp-contract=off`` (the kernels' reduction order names every fused
multiply-add explicitly) and without packed-fp32 instructions.  The host-only
ABI file is compiled with g++.  Objects go to ``modulate_ln_amd/_build/``;
the shared library lands next to this file, where the binding loads it.
"""

from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
INCLUDE = os.path.join(os.path.dirname(HERE), "include")
LIB = os.path.join(HERE, "libadaln.so")

HIP_SOURCES = [
    "ln_modulate.hip",
    "residual_gate_add.hip",
    "qk_head_layernorm.hip",
    "bias_gelu_tanh.hip",
    "residual_ln_modulate.hip",
    "modulate_scale_shift.hip",
    "temb_table_slices.hip",
]
HOST_SOURCES = ["abi.cpp"]

ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
HIPCC = os.path.join(ROCM, "bin", "hipcc")

HIP_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-ffp-contract=off",
    "-fno-fast-math",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
    "-Wno-unused-command-line-argument",
    "-I", INCLUDE,
]
HOST_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-Wall", "-Wextra", "-I", INCLUDE]


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if r.returncode != 0:
        raise RuntimeError("build step failed (%d): %s\n%s" % (r.returncode, " ".join(cmd), r.stdout))
    return r.stdout


def _obj(src: str) -> str:
    return os.path.join(BUILD, os.path.splitext(src)[0] + ".o")


def build(verbose: bool = False, jobs: int = 8) -> str:
    """Compile every source (always, also when a library is present) and link."""
    if not os.path.exists(HIPCC):
        raise RuntimeError("hipcc not found at %s" % HIPCC)
    os.makedirs(BUILD, exist_ok=True)
    cmds = []
    for s in HIP_SOURCES:
        cmds.append([HIPCC, *HIP_FLAGS, "-c", os.path.join(CSRC, s), "-o", _obj(s)])
    for s in HOST_SOURCES:
        cmds.append(["g++", *HOST_FLAGS, "-c", os.path.join(CSRC, s), "-o", _obj(s)])
    with cf.ThreadPoolExecutor(max_workers=max(1, min(jobs, len(cmds)))) as ex:
        for out in ex.map(_run, cmds):
            if verbose and out.strip():
                print(out)
    tmp = LIB + ".tmp%d" % os.getpid()
    objs = [_obj(s) for s in HIP_SOURCES + HOST_SOURCES]
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs])
    os.replace(tmp, LIB)
    return LIB


def clean() -> None:
    shutil.rmtree(BUILD, ignore_errors=True)


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
