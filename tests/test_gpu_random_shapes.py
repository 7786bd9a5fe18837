"""Seeded random shapes and layouts through every entry point, each result compared with the
oracle -- bit for bit in the order the library reports (GELU: within one bf16 ulp of the fp64
oracle).  Row lengths cover every kernel family (one wave, several waves, ragged last steps,
8-byte vectors), storage covers contiguous, padded, misaligned, sample-padded and transposed
views, and several samples with their own adaLN rows.  The draws come from the seed alone, so
every case is reproducible from its id.  A second set draws thousands of rows (around one row
per wave of the launch) for the norm kernels and the fused update."""

from __future__ import annotations

import numpy as np
import pytest
import torch

from test_gpu_fused import run_fused
from test_gpu_modulate import run_mod
from test_gpu_parity import DEV, check_gelu, rand_bf16, run_ln, run_qk, run_rga
from test_gpu_quant import run_fold, run_fp8
from test_gpu_rms import run_qk_rms, run_rms

pytestmark = pytest.mark.gpu

LAYOUTS = ("contiguous", "padded", "misaligned", "sample_padded", "transposed")


@pytest.fixture(scope="module")
def ops():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import modulate_ln_amd as m

    m._native.lib()  # fail loudly if the library is missing
    return m


def draw_D(r: np.random.Generator) -> int:
    """A hidden size (multiple of 4) from one of the row-length classes."""
    cls = r.integers(0, 5)
    if cls == 0:
        return 4 * int(r.integers(1, 129))  # short rows, one wave, often a partial step
    if cls == 1:
        return 4 * int(r.integers(129, 1025))  # up to 4096, one wave, several steps
    if cls == 2:
        return int(r.choice([2240, 3072, 4096, 4092, 4100]))
    if cls == 3:
        return 4 * int(r.integers(1025, 4097))  # 2 and 4 waves per row
    return 4 * int(r.integers(4097, 5121))  # up to 20480: 8 waves per row


def draw_rows(r: np.random.Generator, D: int):
    """(B, S) with at most about 2^20 elements in all."""
    B = int(r.integers(1, 4))
    smax = max(1, (1 << 20) // (B * D))
    S = int(r.integers(1, min(smax, 300) + 1))
    return B, S


def make_x(r: np.random.Generator, g: torch.Generator, layout: str, B: int, S: int, D: int):
    std, mean = float(r.choice([0.5, 1.0, 3.0])), float(r.choice([0.0, 0.5, -2.0]))
    if layout == "padded":
        pad = int(r.choice([8, 24]))
        return rand_bf16((B, S, D + pad), g, std=std, mean=mean).to(DEV)[:, :, :D]
    if layout == "misaligned":
        return rand_bf16((B, S, D + 4), g, std=std, mean=mean).to(DEV)[:, :, 1:1 + D]
    if layout == "sample_padded":
        return rand_bf16((B, S + 3, D), g, std=std, mean=mean).to(DEV)[:, :S]
    if layout == "transposed":
        return rand_bf16((B, D, S), g, std=std, mean=mean).to(DEV).transpose(1, 2)
    return rand_bf16((B, S, D), g, std=std, mean=mean).to(DEV)


@pytest.mark.parametrize("seed", range(30))
def test_norm_family_random(ops, orc, seed):
    """ln_modulate (with and without statistics; with a workspace on transposed storage),
    RMSNorm, the FP8 producer, the fold and the bare modulation on one random case."""
    r = np.random.default_rng(1000 + seed)
    g = torch.Generator().manual_seed(1000 + seed)
    D = draw_D(r)
    B, S = draw_rows(r, D)
    layout = LAYOUTS[int(r.integers(0, len(LAYOUTS)))]
    if layout == "transposed" and r.random() < 0.5:
        S = 64 * int(r.integers(1, 5))  # whole 8- and 64-token groups (tiles, workspace path)
    x = make_x(r, g, layout, B, S, D)
    sc = rand_bf16((B, D), g, std=0.1).to(DEV)
    sh = rand_bf16((B, D), g, std=0.1).to(DEV)
    eps = float(r.choice([1e-6, 1e-5]))
    what = "seed %d: %s (%d,%d,%d)" % (seed, layout, B, S, D)
    y = run_ln(ops, orc, x, sc, sh, eps, stats=bool(r.random() < 0.7), check_fp64=False, what=what)
    if layout == "transposed":
        ws = ops.ln_modulate_workspace(x)
        for _ in range(2):  # the workspace is reused as it is left
            y2 = ops.ln_modulate(x, sc, sh, eps, workspace=ws)
            torch.cuda.synchronize()
            assert torch.equal(y2.view(torch.int16), y.view(torch.int16)), "workspace " + what
    run_rms(ops, orc, x, sc, sh, eps, check_fp64=False, what=what)
    run_fp8(ops, orc, x, sc, sh, eps, float(r.choice([0.01, 0.25, 1.0])), what)
    run_fold(ops, orc, x, sc, sh, eps, what)
    if layout != "transposed":  # the bare modulation takes rows of unit stride
        run_mod(ops, orc, x, sc, sh, what=what)


@pytest.mark.parametrize("seed", range(12))
def test_norm_family_random_many_rows(ops, orc, seed):
    """Thousands of rows of up to 4096 elements (around and past one row per wave of the
    launch, where the launch shapes switch: prefetching blocks past one row per wave of the
    16-wave shape, launches sized to the blocks a compute unit holds): LayerNorm, RMSNorm,
    the FP8 producer and, on vector-aligned rows, the fused update."""
    r = np.random.default_rng(5000 + seed)
    g = torch.Generator().manual_seed(5000 + seed)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    D = int(r.choice([4 * int(r.integers(257, 1025)), int(r.choice([2240, 3072, 3584, 3840, 4000, 4096]))]))
    B = int(r.integers(1, 3))
    S = (int(r.integers(12 * cus, 24 * cus)) + B - 1) // B
    x = make_x(r, g, "contiguous" if r.random() < 0.7 else "padded", B, S, D)
    sc = rand_bf16((B, D), g, std=0.1).to(DEV)
    sh = rand_bf16((B, D), g, std=0.1).to(DEV)
    what = "seed %d: (%d,%d,%d)" % (seed, B, S, D)
    run_ln(ops, orc, x, sc, sh, 1e-6, stats=True, check_fp64=False, what=what)
    run_rms(ops, orc, x, sc, sh, 1e-6, check_fp64=False, what=what)
    run_fp8(ops, orc, x, sc, sh, 1e-6, 0.05, what)
    if D % 8 == 0:
        upd = rand_bf16((B, S, D), g).to(DEV)
        gate = rand_bf16((B, D), g, std=0.5).to(DEV)
        run_fused(ops, orc, x.contiguous(), gate, upd, sc, sh, 1e-6, what=what)


@pytest.mark.parametrize("seed", range(16))
def test_residual_family_random(ops, orc, seed):
    """residual_gate_add and the fused update with ln_modulate on one random case (the fused
    entry point on vector-aligned rows; residual_gate_add also on misaligned ones)."""
    r = np.random.default_rng(2000 + seed)
    g = torch.Generator().manual_seed(2000 + seed)
    D = draw_D(r)
    B, S = draw_rows(r, D)
    layout = LAYOUTS[int(r.integers(0, 4))]  # residual rows with unit stride along D
    res = make_x(r, g, layout, B, S, D)
    upd = rand_bf16((B, S, D), g).to(DEV)
    gate = rand_bf16((B, D), g, std=0.5).to(DEV)
    sc = rand_bf16((B, D), g, std=0.1).to(DEV)
    sh = rand_bf16((B, D), g, std=0.1).to(DEV)
    what = "seed %d: %s (%d,%d,%d)" % (seed, layout, B, S, D)
    run_rga(ops, orc, res, gate, upd, what=what)
    if layout != "misaligned":  # vector-aligned rows: the fused kernels' order is the rows' order
        run_fused(ops, orc, res, gate, upd, sc, sh, float(r.choice([1e-6, 1e-5])), what=what)


@pytest.mark.parametrize("seed", range(16))
def test_qk_family_random(ops, orc, seed):
    """Per-head LayerNorm (affine or not) and RMSNorm of q and k on one random case: contiguous
    heads, heads read out of a packed [B,S,3,H,Dh] projection, or one head per token."""
    r = np.random.default_rng(3000 + seed)
    g = torch.Generator().manual_seed(3000 + seed)
    Dh = 4 * int(r.integers(1, 65))
    B, S = int(r.integers(1, 3)), int(r.integers(1, 200))
    H = int(r.choice([1, 3, 8, 32]))
    kind = int(r.integers(0, 2))
    if kind == 0:
        q = rand_bf16((B, S, H, Dh), g).to(DEV)
        k = rand_bf16((B, S, H, Dh), g, std=2.0).to(DEV)
    else:
        qkv = rand_bf16((B, S, 3, H, Dh), g).to(DEV)
        q, k = qkv[:, :, 0], qkv[:, :, 1]
    w = tuple(rand_bf16((Dh,), g, mean=m, std=s).to(DEV) for m, s in ((1, .05), (0, .02), (1, .05), (0, .02)))
    what = "seed %d: kind %d (%d,%d,%d,%d)" % (seed, kind, B, S, H, Dh)
    run_qk(ops, orc, q, k, w if r.random() < 0.7 else None, 1e-6, what=what)
    run_qk_rms(ops, orc, q, k, (w[0], w[2]) if r.random() < 0.7 else None, 1e-6, what=what)


@pytest.mark.parametrize("seed", range(8))
def test_gelu_random(ops, orc, seed):
    r = np.random.default_rng(4000 + seed)
    g = torch.Generator().manual_seed(4000 + seed)
    width = int(r.integers(1, 20000))
    rows = int(r.integers(1, max(2, (1 << 20) // width)))
    x = rand_bf16((rows, width), g, std=float(r.choice([1.0, 3.0, 8.0]))).to(DEV)
    bias = rand_bf16((width,), g, std=0.5).to(DEV)
    check_gelu(ops, orc, x, bias, "seed %d: (%d,%d)" % (seed, rows, width))
