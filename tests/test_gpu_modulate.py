"""Parity of modulate_scale_shift and temb_table_slices with the CPU oracle,
through the C ABI.

Bar: bit-exact (modulate_scale_shift: the three eager bf16 roundings;
temb_table_slices: one fp32 addition per element, compared as bit patterns).
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

from modulate_ln_amd import workloads as W

from test_gpu_parity import DEV, FP32, assert_bits_equal, bits, device_normal_bf16, rand_bf16

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ops():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import modulate_ln_amd as m

    m._native.lib()
    return m


def run_mod(ops, orc, x, sc, sh, *, out=None, what=""):
    B, S, D = x.shape
    per_token = sc.dim() == 3 and sc.shape[1] == S and S != 1

    def rows(t):
        if per_token:
            return bits(t.expand(B, S, D).contiguous().reshape(B * S, D))
        t2 = t[:, 0] if t.dim() == 3 else t
        return bits(t2.expand(B, D))

    y = ops.modulate_scale_shift(x, sc, sh, out=out)
    torch.cuda.synchronize()
    want = orc.modulate_scale_shift(bits(x.contiguous().reshape(B * S, D)), rows(sc), rows(sh), S, FP32)
    assert_bits_equal(bits(y.reshape(B * S, D)), want, "modulate_scale_shift " + what)
    return y


def test_modulate_glm_square_shape(ops, orc):
    wl = W.glm_square()
    t = {k: v.to(DEV) for k, v in wl.tensors.items()}
    run_mod(ops, orc, t["x"], t["scale"], t["shift"], what="(1,4096,4096) per sample")
    g = torch.Generator().manual_seed(50)
    sc = rand_bf16((1, 4096, 4096), g, std=0.1).to(DEV)
    sh = rand_bf16((1, 4096, 4096), g, std=0.1).to(DEV)
    run_mod(ops, orc, t["x"], sc, sh, what="(1,4096,4096) per token")


def test_modulate_large_per_sample(ops, orc):
    """(2,4096,4096) = 2^25 elements: the one-shot grid with per-sample rows."""
    g = torch.Generator().manual_seed(52)
    x = rand_bf16((2, 4096, 4096), g).to(DEV)
    sc = rand_bf16((2, 4096), g, std=0.1).to(DEV)
    sh = rand_bf16((2, 4096), g, std=0.1).to(DEV)
    run_mod(ops, orc, x, sc, sh, what="(2,4096,4096) per sample")


def test_modulate_row_beyond_2g_elements(ops, orc):
    """One row of 2^31 + 4096 elements (the one-shot grid, 2 GiB+ per tensor): element offsets
    pass 2^31, so its indexing must be 64-bit.  The oracle checks the first and the last 8192
    elements (the op is element-wise)."""
    D = (1 << 31) + 4096
    x = device_normal_bf16((1, 1, D), 11)
    sc = device_normal_bf16((1, 1, D), 12, std=0.1)
    sh = device_normal_bf16((1, 1, D), 13, std=0.1)
    y = ops.modulate_scale_shift(x, sc, sh)
    torch.cuda.synchronize()
    for lo in (0, D - 8192):
        sl = slice(lo, lo + 8192)
        want = orc.modulate_scale_shift(bits(x[0, :, sl]), bits(sc[0, :, sl]), bits(sh[0, :, sl]), 1, FP32)
        assert_bits_equal(bits(y[0, :, sl]), want, "modulate beyond 2^31 at %d" % lo)
    del x, sc, sh, y
    torch.cuda.empty_cache()


@pytest.mark.parametrize("D", [1, 3, 4, 8, 520, 2240, 4096, 4100, 12288])
@pytest.mark.parametrize("per_token", [False, True])
def test_modulate_hidden_sizes(ops, orc, D, per_token):
    g = torch.Generator().manual_seed(600 + D)
    B, S = 2, 9
    x = rand_bf16((B, S, D), g, std=3.0).to(DEV)
    shape = (B, S, D) if per_token else (B, D)
    sc = rand_bf16(shape, g, std=0.5).to(DEV)
    sh = rand_bf16(shape, g, std=0.5).to(DEV)
    run_mod(ops, orc, x, sc, sh, what="D=%d per_token=%s" % (D, per_token))


def test_modulate_views_inplace_special(ops, orc):
    g = torch.Generator().manual_seed(51)
    B, S, D = 2, 17, 3072
    x = rand_bf16((B, S, D), g).to(DEV)
    emb = rand_bf16((B, 6, D), g, std=0.1).to(DEV)
    ref = run_mod(ops, orc, x, emb[:, 1], emb[:, 0], what="adaLN chunk views")
    x2 = x.clone()
    ops.modulate_scale_shift(x2, emb[:, 1], emb[:, 0], out=x2)
    assert torch.equal(x2.view(torch.int16), ref.view(torch.int16))
    one = rand_bf16((1, D), g, std=0.1).to(DEV)
    run_mod(ops, orc, x, one, one, what="one row for all samples")
    big = rand_bf16((B, S, D + 1), g).to(DEV)
    run_mod(ops, orc, big[:, :, 1:], emb[:, 1], emb[:, 0], what="misaligned x")
    xt = rand_bf16((B, S, 2 * D), g).to(DEV)[:, :, :D]  # padded rows
    tok = rand_bf16((B, S, D), g, std=0.1).to(DEV)
    run_mod(ops, orc, xt, tok, emb[:, 0:1], what="padded x, per-token scale, per-sample shift")
    xs = x.clone()
    xs[0, 3, 5] = float("nan")
    y = ops.modulate_scale_shift(xs, emb[:, 1], emb[:, 0])
    torch.cuda.synchronize()
    assert torch.isnan(y[0, 3, 5]) and torch.isnan(y).sum() == 1
    buf = torch.empty(B * S * D + 8, dtype=torch.bfloat16, device=DEV)
    xin, xout = buf[8:].view(B, S, D), buf[:B * S * D].view(B, S, D)
    with pytest.raises(ops.AdalnError):  # output overlapping the input other than exactly
        ops.modulate_scale_shift(xin, emb[:, 1], emb[:, 0], out=xout)


def run_temb(ops, orc, table, temb, what=""):
    out = ops.temb_table_slices(table, temb)
    torch.cuda.synchronize()
    f32 = temb.dtype == torch.float32
    t_in = temb.contiguous().cpu().numpy() if f32 else bits(temb.contiguous())
    want = orc.temb_table_slices(table.reshape(-1, table.shape[-1]).cpu().numpy(), t_in, temb_is_f32=f32)
    got = out.cpu().numpy()
    assert got.shape == want.shape
    bad = np.argwhere(got.view(np.uint32) != want.view(np.uint32))
    assert bad.size == 0, "temb_table_slices %s: %d mismatches, first at %s" % (what, len(bad), bad[0])
    return out


@pytest.mark.parametrize("D", [1, 8, 64, 520, 3072, 4100, 5120])
@pytest.mark.parametrize("nmod", [1, 6, 9])
def test_temb_shapes(ops, orc, D, nmod):
    g = torch.Generator().manual_seed(700 + 10 * D + nmod)
    table = (torch.randn(nmod, D, generator=g) * 0.1).to(DEV)
    temb = rand_bf16((2, 13, nmod, D), g).to(DEV)
    run_temb(ops, orc, table, temb, "bf16 D=%d nmod=%d" % (D, nmod))
    temb32 = torch.randn(2, 13, nmod, D, generator=g).to(DEV)
    run_temb(ops, orc, table, temb32, "fp32 D=%d nmod=%d" % (D, nmod))


def test_temb_views(ops, orc):
    g = torch.Generator().manual_seed(52)
    D, M = 3072, 6
    table = (torch.randn(1, M, D, generator=g) * 0.1).to(DEV)  # leading singleton dim, as the model's
    big = rand_bf16((2, 11, M + 2, D), g).to(DEV)
    run_temb(ops, orc, table, big[:, :, 1:M + 1], "slice of a wider embedding")
    odd = rand_bf16((2, 11, M, D + 1), g).to(DEV)
    run_temb(ops, orc, table, odd[..., 1:], "misaligned temb")


def test_temb_wan_shape_sampled_rows(ops, orc):
    """(1,109120,6,3072): the full size (8 GB of fp32 out); sampled token rows against the
    oracle, every slice."""
    wl = W.wan_temb()
    table = wl.tensors["table"].to(DEV)
    frame = wl.tensors["temb_frame"]
    temb = W.tile(frame.to(DEV), wl.meta["frames"])
    out = ops.temb_table_slices(table, temb)
    torch.cuda.synchronize()
    Lt = temb.shape[1]
    rows = torch.linspace(0, Lt - 1, 7).long()
    tpf = frame.shape[1]  # token l of the tiled embedding is token l % tpf of the frame
    want = orc.temb_table_slices(wl.tensors["table"].numpy(), bits(frame[:, rows % tpf]))
    got = out[:, :, rows.to(DEV)].cpu().numpy()
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))
    del out, temb
