"""Parity of residual_gate_add_ln_modulate (the gated residual update fused
with ln_modulate of its result) with the CPU oracle, through the C ABI.

Bar: both outputs (the new residual and the modulated norm) and the fp32
statistics bit-exact against the oracle's fixed-order fp32 mode, run in the
order the library reports (adaln_order_for), and bit-identical to the two
unfused entry points run back to back.
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

from modulate_ln_amd import workloads as W

from test_gpu_parity import DEV, FP32, N_OP_FUSED, N_OP_LN, assert_bits_equal, bits, gpu_chain, oracle_chain_rows, order, rand_bf16

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ops():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import modulate_ln_amd as m

    m._native.lib()
    return m


def rows2d(t, B, D):
    """[B,D] / [B,1,D] / broadcast [1,D] adaLN rows -> [B,D] bits"""
    if t.dim() == 3:
        t = t[:, 0]
    return bits(t.expand(B, D))


def run_fused(ops, orc, res, gate, upd, scale, shift, eps, *, what="", residual_out=None, out=None, stats=True):
    B, S, D = res.shape
    R = B * S
    res_b = bits(res.contiguous().reshape(R, D))
    upd_b = bits(upd.contiguous().reshape(R, D))
    g_b, sc_b, sh_b = rows2d(gate, B, D), rows2d(scale, B, D), rows2d(shift, B, D)
    mean = torch.empty(R, dtype=torch.float32, device=DEV) if stats else None
    rstd = torch.empty(R, dtype=torch.float32, device=DEV) if stats else None
    xo, y = ops.residual_gate_add_ln_modulate(res, gate, upd, scale, shift, eps, residual_out=residual_out,
                                              out=out, mean_out=mean, rstd_out=rstd)
    torch.cuda.synchronize()
    V, L = order(N_OP_FUSED, D, res)
    assert order(N_OP_FUSED, D, upd) == (V, L) == order(N_OP_LN, D, res)
    want_x, want_y, m32, r32 = orc.residual_gate_add_ln_modulate(res_b, g_b, upd_b, sc_b, sh_b, S, eps, FP32,
                                                                 V=V, L=L)
    assert_bits_equal(bits(xo.reshape(R, D)), want_x, "residual_out " + what)
    assert_bits_equal(bits(y.reshape(R, D)), want_y, "out " + what)
    if stats:
        assert np.array_equal(mean.cpu().numpy().astype(np.float64), m32), "mean " + what
        assert np.array_equal(rstd.cpu().numpy().astype(np.float64), r32), "rstd " + what
    return xo, y


def test_fused_glm_square_config(ops, orc):
    """(1,4096,4096) with 1% x20 outliers, eps 1e-5, full size."""
    wl = W.glm_square()
    t = {k: v.to(DEV) for k, v in wl.tensors.items()}
    run_fused(ops, orc, t["x"], t["gate"], t["update"], t["scale"], t["shift"], wl.meta["eps"],
              what="(1,4096,4096)")


@pytest.mark.parametrize("D", [4, 8, 12, 60, 64, 520, 1000, 2240, 3072, 4096, 4100, 8192, 8200, 12288])
def test_fused_hidden_sizes(ops, orc, D):
    g = torch.Generator().manual_seed(700 + D)
    B, S = 2, 37
    res = rand_bf16((B, S, D), g, mean=0.5).to(DEV)
    upd = rand_bf16((B, S, D), g, std=3.0).to(DEV)
    emb = rand_bf16((B, 6, D), g, std=0.1).to(DEV)
    run_fused(ops, orc, res, emb[:, 2], upd, emb[:, 1], emb[:, 0], 1e-6, what="D=%d" % D)


@pytest.mark.parametrize("D,W", [(8192, 2), (4100, 2), (12296, 4), (32768, 8), (65536, 16), (65532, 16)])
def test_fused_waves_per_row(ops, orc, D, W):
    """Rows of W > 1 waves take one fused launch (the cross-wave merge through LDS) and match
    the oracle in the order the library reports."""
    from modulate_ln_amd import _native as N

    assert N.order_for(N.OP_RESIDUAL_GATE_ADD_LN_MODULATE, D).W == W
    g = torch.Generator().manual_seed(D + 3)
    B, S = 2, 3
    res = rand_bf16((B, S, D), g, std=2.0).to(DEV)
    upd = rand_bf16((B, S, D), g).to(DEV)
    gate = rand_bf16((B, D), g, std=0.5).to(DEV)
    sc = rand_bf16((B, D), g, std=0.1).to(DEV)
    sh = rand_bf16((B, D), g, std=0.1).to(DEV)
    run_fused(ops, orc, res, gate, upd, sc, sh, 1e-6, what="W=%d D=%d" % (W, D))
    # padded rows (still vector-aligned): the fused kernel reads strided rows
    bigr = rand_bf16((B, S, D + 16), g).to(DEV)
    run_fused(ops, orc, bigr[:, :, 8:8 + D], gate, upd, sc, sh, 1e-5, what="strided W=%d D=%d" % (W, D))


@pytest.mark.parametrize("D,S", [(4096, 64), (3584, 64), (3584, 300), (4096, 1024), (4096, 2048)])
def test_fused_few_long_rows(ops, orc, D, S):
    """Rows of 7-8 full vector steps, too few to fill the compute units with 16-wave blocks:
    one wave per row in blocks of their own (same lanes and merges)."""
    g = torch.Generator().manual_seed(3 * D + S)
    res = rand_bf16((1, S, D), g, std=2.0).to(DEV)
    upd = rand_bf16((1, S, D), g).to(DEV)
    gate = rand_bf16((1, D), g, std=0.5).to(DEV)
    sc = rand_bf16((1, D), g, std=0.1).to(DEV)
    sh = rand_bf16((1, D), g, std=0.1).to(DEV)
    run_fused(ops, orc, res, gate, upd, sc, sh, 1e-6, what="few rows (1,%d,%d)" % (S, D))


@pytest.mark.parametrize("B,S,D", [(1, 4096, 2048), (1, 4096, 2240), (2, 2000, 3072)])
def test_fused_held_blocks(ops, orc, B, S, D):
    """One row per wave at the shape's own sizing, more blocks than a compute unit holds
    (registers): the launch is sized to what is held, so some waves walk two rows."""
    g = torch.Generator().manual_seed(7 * D + S + B)
    res = rand_bf16((B, S, D), g, std=2.0).to(DEV)
    upd = rand_bf16((B, S, D), g).to(DEV)
    gate = rand_bf16((B, D), g, std=0.5).to(DEV)
    sc = rand_bf16((B, D), g, std=0.1).to(DEV)
    sh = rand_bf16((B, D), g, std=0.1).to(DEV)
    run_fused(ops, orc, res, gate, upd, sc, sh, 1e-6, what="held blocks (%d,%d,%d)" % (B, S, D))


@pytest.mark.parametrize("D,B", [(4096, 1), (3584, 2), (4096, 3)])
def test_fused_many_long_rows(ops, orc, D, B):
    """More rows of 7-8 full vector steps than 16-wave blocks hold at one per wave: 4-wave
    blocks (same lanes and merges); ragged last blocks, several samples."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    S = (16 * cus + 123 + B - 1) // B
    g = torch.Generator().manual_seed(5 * D + S + B)
    res = rand_bf16((B, S, D), g, std=2.0).to(DEV)
    upd = rand_bf16((B, S, D), g).to(DEV)
    gate = rand_bf16((B, D), g, std=0.5).to(DEV)
    sc = rand_bf16((B, D), g, std=0.1).to(DEV)
    sh = rand_bf16((B, D), g, std=0.1).to(DEV)
    run_fused(ops, orc, res, gate, upd, sc, sh, 1e-6, what="many rows (%d,%d,%d)" % (B, S, D))


@pytest.mark.parametrize("D,W", [(8192, 2), (5120, 2), (16384, 4), (12296, 4)])
@pytest.mark.parametrize("B,S", [(1, None), (1, "half"), (3, 9)])
def test_fused_waves_per_row_shared_tables(ops, orc, D, W, B, S):
    """Enough rows of up to 16384 elements: blocks of 16 waves hold 16 / W rows of one sample
    and build its tables once (whole blocks, then a partial last block per sample); with few
    rows (S given), one row per block.  Both outputs and the statistics match the oracle, on
    contiguous and padded rows."""
    from modulate_ln_amd import _native as N
    from test_gpu_parity import shared_table_rows

    assert N.order_for(N.OP_RESIDUAL_GATE_ADD_LN_MODULATE, D).W == W
    S = shared_table_rows(W, B, half=True) if S == "half" else (S if S is not None else shared_table_rows(W, B))
    g = torch.Generator().manual_seed(5 * D + S)
    res = rand_bf16((B, S, D), g, std=2.0).to(DEV)
    upd = rand_bf16((B, S, D), g).to(DEV)
    gate = rand_bf16((B, D), g, std=0.5).to(DEV)
    sc = rand_bf16((B, D), g, std=0.1).to(DEV)
    sh = rand_bf16((B, D), g, std=0.1).to(DEV)
    run_fused(ops, orc, res, gate, upd, sc, sh, 1e-6, what="shared tables W=%d D=%d (%d,%d)" % (W, D, B, S))
    bigr = rand_bf16((B, S, D + 16), g).to(DEV)
    run_fused(ops, orc, bigr[:, :, 8:8 + D], gate, upd, sc, sh, 1e-5,
              what="shared tables strided W=%d D=%d (%d,%d)" % (W, D, B, S))


@pytest.mark.parametrize("B,S", [(1, 1), (3, 1), (1, 5), (3, 37), (2, 1024), (5, 301)])
def test_fused_rows(ops, orc, B, S):
    g = torch.Generator().manual_seed(31 * B + S)
    D = 3072
    res = rand_bf16((B, S, D), g).to(DEV)
    upd = rand_bf16((B, S, D), g).to(DEV)
    gate, sc, sh = (rand_bf16((B, D), g, std=0.1).to(DEV) for _ in range(3))
    run_fused(ops, orc, res, gate, upd, sc, sh, 1e-6, what="B=%d S=%d" % (B, S))


def test_fused_equals_unfused_and_inplace(ops, orc):
    g = torch.Generator().manual_seed(41)
    B, S, D = 2, 129, 2240
    res = rand_bf16((B, S, D), g).to(DEV)
    upd = rand_bf16((B, S, D), g, std=2.0).to(DEV)
    emb = rand_bf16((B, 6, D), g, std=0.1).to(DEV)
    gate, sc, sh = emb[:, 2], emb[:, 4], emb[:, 3]
    xo, y = run_fused(ops, orc, res, gate, upd, sc, sh, 1e-6, what="reference")
    # the unfused pair gives the same bits
    x2 = ops.residual_gate_add(res, gate, upd)
    y2 = ops.ln_modulate(x2, sc, sh, 1e-6)
    assert torch.equal(x2.view(torch.int16), xo.view(torch.int16))
    assert torch.equal(y2.view(torch.int16), y.view(torch.int16))
    # in place: new residual over the residual, output over the update
    r3, u3 = res.clone(), upd.clone()
    ops.residual_gate_add_ln_modulate(r3, gate, u3, sc, sh, 1e-6, residual_out=r3, out=u3)
    assert torch.equal(r3.view(torch.int16), xo.view(torch.int16))
    assert torch.equal(u3.view(torch.int16), y.view(torch.int16))


def test_fused_views_and_fallback_layouts(ops, orc):
    g = torch.Generator().manual_seed(43)
    B, S, D = 2, 33, 1024
    # padded residual rows (fused kernel), one adaLN row broadcast to both samples
    bigr = rand_bf16((B, S, D + 8), g).to(DEV)
    upd = rand_bf16((B, S, D), g).to(DEV)
    one = rand_bf16((1, D), g, std=0.1).to(DEV)
    sc, sh = rand_bf16((B, 1, D), g, std=0.1).to(DEV), rand_bf16((B, 1, D), g, std=0.1).to(DEV)
    run_fused(ops, orc, bigr[:, :, :D], one, upd, sc, sh, 1e-6, what="padded residual")
    # misaligned update rows: the two unfused kernels run back to back
    bigu = rand_bf16((B, S, D + 1), g).to(DEV)
    run_fused(ops, orc, bigr[:, :, :D], one, bigu[:, :, 1:], sc, sh, 1e-6, what="misaligned update")
    # rows longer than the fused kernel's LDS plan
    D2 = 16384
    res = rand_bf16((1, 9, D2), g).to(DEV)
    upd = rand_bf16((1, 9, D2), g).to(DEV)
    e = rand_bf16((1, 3, D2), g, std=0.1).to(DEV)
    run_fused(ops, orc, res, e[:, 0], upd, e[:, 1], e[:, 2], 1e-6, what="D=16384")


def test_fused_special_values(ops, orc):
    D = 512
    g = torch.Generator().manual_seed(47)
    res = rand_bf16((1, 4, D), g).to(DEV)
    upd = rand_bf16((1, 4, D), g).to(DEV)
    z = torch.zeros(1, D, dtype=torch.bfloat16, device=DEV)
    # gate 0 and a -0 residual: new residual +0; constant rows normalize to +0
    res[0, 0] = -0.0
    res[0, 1] = 3.0
    upd[0, :2] = upd[0, :2].abs()
    xo, y = run_fused(ops, orc, res, z, upd, z, z, 1e-6, what="zeros")
    assert torch.all(xo[0, 0].view(torch.int16) == 0)
    assert torch.all(y[0, :2].view(torch.int16) == 0)
    # a NaN in the update poisons that row's output (and that residual element)
    upd[0, 2, 7] = float("nan")
    xo, y = ops.residual_gate_add_ln_modulate(res, torch.ones_like(z), upd, z, z, 1e-6)
    torch.cuda.synchronize()
    assert torch.isnan(xo[0, 2, 7]) and torch.isnan(y[0, 2]).all()
    assert not torch.isnan(y[0, 3]).any()


def test_fused_empty_and_errors(ops):
    z = torch.zeros(2, 0, 8, dtype=torch.bfloat16, device=DEV)
    r = torch.zeros(2, 8, dtype=torch.bfloat16, device=DEV)
    xo, y = ops.residual_gate_add_ln_modulate(z, r, z, r, r, 1e-6)
    assert xo.shape == (2, 0, 8) and y.shape == (2, 0, 8)
    x = torch.zeros(1, 4, 8, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(ops.AdalnError):  # out over the residual
        ops.residual_gate_add_ln_modulate(x, r[:1], x.clone(), r[:1], r[:1], 1e-6, out=x)
    with pytest.raises(ops.AdalnError):  # D % 4 != 0
        x6 = torch.zeros(1, 4, 6, dtype=torch.bfloat16, device=DEV)
        r6 = torch.zeros(1, 6, dtype=torch.bfloat16, device=DEV)
        ops.residual_gate_add_ln_modulate(x6, r6, x6, r6, r6, 1e-6)


def gpu_chain_fused(ops, x, embs_dev, eps):
    """The DiT chain with each gated residual add fused into the LayerNorm that
    reads its result: one ln_modulate, 2*blocks - 1 fused calls, one gate-add."""
    h = torch.empty_like(x)
    e0 = embs_dev[0]
    ops.ln_modulate(x, e0[:, 1], e0[:, 0], eps, out=h)
    for i, emb in enumerate(embs_dev):
        ops.residual_gate_add_ln_modulate(x, emb[:, 2], h, emb[:, 4], emb[:, 3], eps, residual_out=x, out=h)
        if i + 1 < len(embs_dev):
            nxt = embs_dev[i + 1]
            ops.residual_gate_add_ln_modulate(x, emb[:, 5], h, nxt[:, 1], nxt[:, 0], eps, residual_out=x, out=h)
        else:
            ops.residual_gate_add(x, emb[:, 5], h, out=x)
    return x


def test_fused_dit_chain_config(ops, orc):
    """20 blocks on x [4,4096,3072]: the fused chain equals the unfused chain bit for
    bit over the whole tensor, and the oracle chain on sampled rows."""
    wl = W.dit_chain()
    x0 = wl.tensors["x"]
    embs = [e.to(DEV) for e in wl.tensors["embs"]]
    xf = gpu_chain_fused(ops, x0.to(DEV).clone(), embs, wl.meta["eps"])
    xu = gpu_chain(ops, x0.to(DEV).clone(), embs, wl.meta["eps"])
    torch.cuda.synchronize()
    assert torch.equal(xf.view(torch.int16), xu.view(torch.int16))
    B, S, D = x0.shape
    rows = torch.linspace(0, S - 1, 4).long()
    for b in (0, B - 1):
        want = oracle_chain_rows(orc, bits(x0[b, rows]), wl.tensors["embs"], b, wl.meta["eps"])
        assert_bits_equal(bits(xf[b, rows.to(DEV)]), want, "fused chain b=%d" % b)
