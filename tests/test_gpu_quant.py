"""Parity of ln_modulate_fp8 (the LayerNorm + modulate output quantized to
static OCP FP8 E4M3) and ln_modulate_fold (the single-rounding affine fold)
with the CPU oracle, through the C ABI.

Bar: bit-exact -- FP8 codes equal (NaN compared as NaN), fold outputs and
statistics equal the oracle's fixed-order fp32 mode.
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

from modulate_ln_amd import workloads as W

from test_gpu_parity import DEV, FP32, N_OP_LN, assert_bits_equal, bits, order, rand_bf16

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ops():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import modulate_ln_amd as m

    m._native.lib()
    return m


def rows2d(t, B, D):
    t = t[:, 0] if t.dim() == 3 else t
    return bits(t.expand(B, D))


def run_fp8(ops, orc, x, sc, sh, eps, qscale, what=""):
    B, S, D = x.shape
    q = torch.tensor([qscale], dtype=torch.float32, device=DEV)
    mean = torch.empty(B * S, dtype=torch.float32, device=DEV)
    rstd = torch.empty(B * S, dtype=torch.float32, device=DEV)
    y = ops.ln_modulate_fp8(x, sc, sh, q, eps, mean_out=mean, rstd_out=rstd)
    torch.cuda.synchronize()
    V, L = order(N_OP_LN, D, x)
    want, m32, r32 = orc.ln_modulate_fp8(bits(x.contiguous().reshape(B * S, D)), rows2d(sc, B, D), rows2d(sh, B, D),
                                         S, eps, qscale, FP32, V=V, L=L)
    got = y.view(torch.uint8).cpu().numpy().reshape(B * S, D)
    nan_w = (want & 0x7F) == 0x7F
    bad = np.argwhere((got != want) & ~nan_w)
    assert bad.size == 0, "ln_modulate_fp8 %s: %d mismatches, first %s got 0x%02x want 0x%02x" % (
        what, len(bad), bad[0], got[tuple(bad[0])], want[tuple(bad[0])])
    assert np.all((got[nan_w] & 0x7F) == 0x7F), what
    assert np.array_equal(mean.cpu().numpy().astype(np.float64), m32, equal_nan=True), what
    assert np.array_equal(rstd.cpu().numpy().astype(np.float64), r32, equal_nan=True), what
    return y


def test_fp8_glm_square_shape(ops, orc):
    """(1,4096,4096) with 1% x20 outliers; qscale 0.02 sends the outliers' outputs past 448 (clamped)."""
    wl = W.glm_square()
    t = {k: v.to(DEV) for k, v in wl.tensors.items()}
    y = run_fp8(ops, orc, t["x"], t["scale"], t["shift"], wl.meta["eps"], 0.02, "(1,4096,4096)")
    assert (y.view(torch.uint8) & 0x7F).eq(0x7E).any()  # some values saturate at 448
    run_fp8(ops, orc, t["x"], t["scale"], t["shift"], wl.meta["eps"], 1.0, "(1,4096,4096) qscale 1")


@pytest.mark.parametrize("D", [4, 12, 64, 520, 2240, 4096, 4100, 8192, 16384, 20000])
def test_fp8_hidden_sizes(ops, orc, D):
    g = torch.Generator().manual_seed(800 + D)
    x = rand_bf16((2, 5, D), g, std=3.0, mean=0.5).to(DEV)
    sc = rand_bf16((2, D), g, std=0.1).to(DEV)
    sh = rand_bf16((2, D), g, std=0.1).to(DEV)
    run_fp8(ops, orc, x, sc, sh, 1e-6, 0.037, "D=%d" % D)


@pytest.mark.parametrize("D,S", [(4096, 64), (3584, 300), (4096, 1024)])
def test_fp8_few_long_rows(ops, orc, D, S):
    """Rows of 7-8 full vector steps, too few to fill the compute units with 16-wave blocks:
    the row kernel takes them (same lanes and merges)."""
    g = torch.Generator().manual_seed(870 + D + S)
    x = rand_bf16((1, S, D), g, std=3.0, mean=0.5).to(DEV)
    sc = rand_bf16((1, D), g, std=0.1).to(DEV)
    sh = rand_bf16((1, D), g, std=0.1).to(DEV)
    run_fp8(ops, orc, x, sc, sh, 1e-6, 0.037, "few rows (1,%d,%d)" % (S, D))


@pytest.mark.parametrize("D,B", [(4096, 1), (3584, 2)])
def test_fp8_many_long_rows(ops, orc, D, B):
    """More rows of 7-8 full vector steps than 16-wave blocks hold at one per wave: 4-wave
    blocks that prefetch the next row (same lanes and merges)."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    S = (16 * cus + 301 + B - 1) // B
    g = torch.Generator().manual_seed(880 + D + S)
    x = rand_bf16((B, S, D), g, std=3.0, mean=0.5).to(DEV)
    sc = rand_bf16((B, D), g, std=0.1).to(DEV)
    sh = rand_bf16((B, D), g, std=0.1).to(DEV)
    run_fp8(ops, orc, x, sc, sh, 1e-6, 0.037, "many rows (%d,%d,%d)" % (B, S, D))


def test_fp8_ragged_rows_held_blocks(ops, orc):
    """Rows with a partial last step, the launch sized to the blocks a compute unit holds."""
    g = torch.Generator().manual_seed(8855)
    x = rand_bf16((1, 5120, 2240), g, std=3.0, mean=0.5).to(DEV)
    sc = rand_bf16((1, 2240), g, std=0.1).to(DEV)
    sh = rand_bf16((1, 2240), g, std=0.1).to(DEV)
    run_fp8(ops, orc, x, sc, sh, 1e-6, 0.037, "held blocks (1,5120,2240)")


@pytest.mark.parametrize("D,W", [(8192, 2), (16384, 4)])
def test_fp8_and_fold_long_rows_shared_tables(ops, orc, D, W):
    """Rows of 2 and 4 waves, enough per sample for blocks of 16 waves sharing the sample's
    tables (a partial last block per sample): the FP8 producer and the fold."""
    from test_gpu_parity import shared_table_rows

    S = shared_table_rows(W, 2)
    g = torch.Generator().manual_seed(850 + D)
    x = rand_bf16((2, S, D), g, std=3.0, mean=0.5).to(DEV)
    sc = rand_bf16((2, D), g, std=0.1).to(DEV)
    sh = rand_bf16((2, D), g, std=0.1).to(DEV)
    run_fp8(ops, orc, x, sc, sh, 1e-6, 0.037, "shared tables D=%d S=%d" % (D, S))
    run_fold(ops, orc, x, sc, sh, 1e-6, "shared tables D=%d S=%d" % (D, S))


def test_fp8_layouts_and_specials(ops, orc):
    g = torch.Generator().manual_seed(81)
    B, S, D = 2, 1024, 2240
    xt = rand_bf16((B, D, S), g).to(DEV)
    emb = rand_bf16((B, 6, D), g, std=0.1).to(DEV)
    run_fp8(ops, orc, xt.transpose(1, 2), emb[:, 5], emb[:, 0], 1e-6, 0.1, "transposed")
    big = rand_bf16((B, 7, D + 3), g).to(DEV)
    run_fp8(ops, orc, big[:, :, 1:D + 1], emb[:, 5], emb[:, 0], 1e-6, 0.1, "misaligned x")
    x = rand_bf16((1, 4, 512), g).to(DEV)
    x[0, 1, 9] = float("nan")
    z = torch.zeros(1, 512, dtype=torch.bfloat16, device=DEV)
    y = run_fp8(ops, orc, x, z, z, 1e-6, 0.5, "nan row")
    assert ((y.view(torch.uint8)[0, 1] & 0x7F) == 0x7F).all()
    # the scale is read on the device at run time: a value changed on the stream between two
    # calls takes effect without a host synchronization
    q = torch.tensor([0.5], dtype=torch.float32, device=DEV)
    x2 = rand_bf16((1, 64, 512), g).to(DEV)
    a = ops.ln_modulate_fp8(x2, z, z, q, 1e-6)
    q.fill_(0.25)
    b = ops.ln_modulate_fp8(x2, z, z, q, 1e-6)
    torch.cuda.synchronize()
    V, L = order(N_OP_LN, 512, x2)
    zb = bits(z)
    for got, qs in ((a, 0.5), (b, 0.25)):
        want, _, _ = orc.ln_modulate_fp8(bits(x2.reshape(64, 512)), zb, zb, 64, 1e-6, qs, FP32, V=V, L=L)
        assert np.array_equal(got.view(torch.uint8).cpu().numpy().reshape(64, 512), want)


def test_fp8_overflowing_variance_row(ops, orc):
    """A row whose fp32 m2 overflows (rstd = 1/sqrt(inf) = 0) while its mean stays finite: one
    element's x - mean is then infinite and its normalized value inf * 0 is NaN, which must reach
    the FP8 output as NaN (as in the oracle) on the tabled, transposed and gather paths."""
    g = torch.Generator().manual_seed(97)
    B, S, D = 1, 8, 512
    big = 3.3895313892515355e38  # largest finite bf16
    x = rand_bf16((B, S, D), g)
    row = torch.zeros(D, dtype=torch.float32)
    row[0] = big          # lane 0's first element (vector 0)
    row[256:] = -big      # vectors 32..63: lanes 32..63
    x[0, 3] = row.to(torch.bfloat16)
    sc = rand_bf16((B, D), g, std=0.1).to(DEV)
    sh = rand_bf16((B, D), g, std=0.1).to(DEV)
    xd = x.to(DEV)
    y = run_fp8(ops, orc, xd, sc, sh, 1e-6, 0.5, "overflowing m2, tabled")
    assert ((y.view(torch.uint8)[0, 3, 0] & 0x7F) == 0x7F).item()
    run_fp8(ops, orc, xd.transpose(1, 2).contiguous().transpose(1, 2), sc, sh, 1e-6, 0.5,
            "overflowing m2, transposed")
    pad = torch.zeros((B, S, D + 1), dtype=torch.bfloat16, device=DEV)
    pad[:, :, 1:] = xd
    run_fp8(ops, orc, pad[:, :, 1:], sc, sh, 1e-6, 0.5, "overflowing m2, gather")


def test_fp8_decodes_within_half_e4m3_ulp_of_bf16_chain(ops):
    """The FP8 output is the bf16 chain output rounded once more: decoded, it lies within half an
    E4M3 ulp (2^-4 relative) of ln_modulate's output divided by qscale."""
    wl = W.glm_square(S=256)
    t = {k: v.to(DEV) for k, v in wl.tensors.items()}
    q = torch.tensor([0.05], dtype=torch.float32, device=DEV)
    y8 = ops.ln_modulate_fp8(t["x"], t["scale"], t["shift"], q, 1e-5).float()
    y = ops.ln_modulate(t["x"], t["scale"], t["shift"], 1e-5).float() / 0.05
    y = y.clamp(-448, 448)
    tiny = y.abs() < 2.0 ** -6 * 2
    assert torch.all(((y8 - y).abs() <= y.abs() * 2.0 ** -4 * 1.0001) | tiny)


def run_fold(ops, orc, x, sc, sh, eps, what=""):
    B, S, D = x.shape
    mean = torch.empty(B * S, dtype=torch.float32, device=DEV)
    rstd = torch.empty(B * S, dtype=torch.float32, device=DEV)
    y = ops.ln_modulate_fold(x, sc, sh, eps, mean_out=mean, rstd_out=rstd)
    torch.cuda.synchronize()
    V, L = order(N_OP_LN, D, x)
    want, m32, r32 = orc.ln_modulate_fold(bits(x.contiguous().reshape(B * S, D)), rows2d(sc, B, D),
                                          rows2d(sh, B, D), S, eps, FP32, V=V, L=L)
    assert_bits_equal(bits(y.reshape(B * S, D)), want, "ln_modulate_fold " + what)
    assert np.array_equal(mean.cpu().numpy().astype(np.float64), m32), what
    return y


@pytest.mark.parametrize("D", [4, 12, 520, 2240, 4096, 4100, 16384])
def test_fold_hidden_sizes(ops, orc, D):
    g = torch.Generator().manual_seed(900 + D)
    x = rand_bf16((2, 5, D), g, std=3.0, mean=0.5).to(DEV)
    sc = rand_bf16((2, D), g, std=0.3).to(DEV)
    sh = rand_bf16((2, D), g, std=0.3).to(DEV)
    run_fold(ops, orc, x, sc, sh, 1e-6, "D=%d" % D)


def test_fold_shapes_and_differs_from_chain(ops, orc):
    wl = W.glm_square()
    t = {k: v.to(DEV) for k, v in wl.tensors.items()}
    y = run_fold(ops, orc, t["x"], t["scale"], t["shift"], wl.meta["eps"], "(1,4096,4096)")
    chain = ops.ln_modulate(t["x"], t["scale"], t["shift"], wl.meta["eps"])
    # a different rounding: many elements differ, each by at most two bf16 ulps of the largest
    # intermediate (the chain rounds x_hat and the product, the fold neither)
    d = (y.float() - chain.float()).abs()
    assert (d > 0).any()
    xh = torch.nn.functional.layer_norm(t["x"].float(), (4096,), eps=wl.meta["eps"])
    big = torch.maximum(torch.maximum((xh * (1 + t["scale"].float())).abs(), t["shift"].float().abs()),
                        chain.float().abs())
    assert torch.all(d <= big * 2 * 2.0 ** -7 + 1e-30)
    g = torch.Generator().manual_seed(91)
    xt = rand_bf16((2, 2240, 1024), g).to(DEV)
    emb = rand_bf16((2, 6, 2240), g, std=0.1).to(DEV)
    run_fold(ops, orc, xt.transpose(1, 2), emb[:, 5], emb[:, 0], 1e-6, "transposed")
