"""Parity of the HIP kernels (through the C ABI) with the CPU oracle.

Bar: bit-exact against the oracle's fixed-order fp32 mode for ln_modulate,
residual_gate_add and qk_head_layernorm, run in the order the library reports
through adaln_order_for (V elements per vector, L = 64 W lanes per row for W
waves, 16 per q/k head); within one bf16 ulp of the fp64 oracle for bias +
tanh-GELU.  The
fp64 mode is checked too, at the tolerances the statistics contract states.
Inputs are the seeded synthetic workloads at full size where the oracle is
fast enough, plus edge shapes (tails, tiny and maximal D, strided and
misaligned views, in-place, empty).
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

from modulate_ln_amd import workloads as W

pytestmark = pytest.mark.gpu

FP32, FP64 = 1, 0
DEV = "cuda"
N_OP_LN, N_OP_QK, N_OP_FUSED, N_OP_RMS, N_OP_QK_RMS = 1, 2, 3, 4, 5  # ADALN_OP_* (include/adaln.h)


@pytest.fixture(scope="module")
def ops():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import modulate_ln_amd as m

    m._native.lib()  # fail loudly if the library is missing
    return m


def row_align(t) -> int:
    """Largest power of two (2..16) dividing the byte address of every row start of t."""
    a = t.data_ptr()
    for st, n in zip(t.stride()[:-1], t.shape[:-1]):
        if n > 1:
            a |= st * t.element_size()
    a |= 16
    return a & -a


def order(op: int, D: int, t=None):
    """(V, L) of the reduction order the library reports for op on rows of D elements
    (adaln_order_for through the C ABI), for the storage of the device view t if given."""
    from modulate_ln_amd import _native as N

    sx_d = t.stride(-1) if t is not None else 1
    o = N.order_for(op, D, sx_d, row_align(t) if t is not None else 16)
    assert o.L == (16 if op in (N.OP_QK_HEAD_LAYERNORM, N.OP_QK_RMSNORM) else 64 * o.W), o.as_dict()
    assert o.map == N.MAP_INTERLEAVED and o.fold == N.FOLD_PAIRWISE, o.as_dict()
    return o.V, o.L


def bits(t):
    return W.bits(t)


def f32(b):
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def rand_bf16(shape, g, std=1.0, mean=0.0):
    return W.normal(shape, g, mean=mean, std=std)


def assert_bits_equal(got, want, what=""):
    got = np.asarray(got)
    want = np.asarray(want)
    assert got.shape == want.shape, (got.shape, want.shape)
    bad = np.argwhere(got != want)
    if bad.size:
        i = tuple(bad[0])
        raise AssertionError("%s: %d mismatches, first at %s: got 0x%04x (%r) want 0x%04x (%r)" % (
            what, len(bad), i, got[i], float(f32(got[i])), want[i], float(f32(want[i]))))


# ---------------------------------------------------------------------------
# ln_modulate
# ---------------------------------------------------------------------------

def run_ln(ops, orc, x_dev, scale_dev, shift_dev, eps, *, stats=True, out=None, check_fp64=True, what=""):
    """Run the kernel on (possibly strided) device views and compare with the oracle."""
    B, S, D = x_dev.shape
    mean = torch.empty(B * S, dtype=torch.float32, device=DEV) if stats else None
    rstd = torch.empty(B * S, dtype=torch.float32, device=DEV) if stats else None
    x_log = bits(x_dev.reshape(B * S, D)) if x_dev.is_contiguous() else bits(x_dev.contiguous().reshape(B * S, D))
    sc = scale_dev[:, 0] if scale_dev.dim() == 3 else scale_dev
    sh = shift_dev[:, 0] if shift_dev.dim() == 3 else shift_dev
    sc_b = bits(sc.expand(B, D))
    sh_b = bits(sh.expand(B, D))
    y = ops.ln_modulate(x_dev, scale_dev, shift_dev, eps, out=out, mean_out=mean, rstd_out=rstd)
    torch.cuda.synchronize()
    V, L = order(N_OP_LN, D, x_dev)
    want, m32, r32 = orc.ln_modulate(x_log, sc_b, sh_b, S, eps, FP32, V=V, L=L)
    assert_bits_equal(bits(y.reshape(B * S, D)), want, "ln_modulate %s" % what)
    if stats:
        assert np.array_equal(mean.cpu().numpy().astype(np.float64), m32), "mean " + what
        assert np.array_equal(rstd.cpu().numpy().astype(np.float64), r32), "rstd " + what
        if check_fp64:
            _, m64, r64 = orc.ln_modulate(x_log, sc_b, sh_b, S, eps, FP64)
            sig = 1.0 / r64
            assert np.all(np.abs(m32 - m64) <= 1e-5 * np.sqrt(m64 ** 2 + sig ** 2)), what
            assert np.all(np.abs(r32 - r64) <= 1e-5 * r64), what
    return y


def test_ln_small_config(ops, orc):
    wl = W.ln_small()
    t = wl.tensors
    run_ln(ops, orc, t["x"].to(DEV), t["scale"].to(DEV), t["shift"].to(DEV), wl.meta["eps"], what="(1,256,512)")


def test_ln_sana_transposed_config(ops, orc):
    wl = W.sana_transposed()
    t = wl.tensors
    xt = t["xt"].to(DEV)
    emb = t["emb"].to(DEV)
    x = xt.transpose(1, 2)  # strides (D*S, 1, S)
    assert x.stride() == (2240 * 1024, 1, 1024)
    y = run_ln(ops, orc, x, emb[:, 5], emb[:, 0], wl.meta["eps"], what="sana transposed")
    # the same logical values stored contiguously give the same bits
    y2 = ops.ln_modulate(x.contiguous(), emb[:, 5], emb[:, 0], wl.meta["eps"])
    assert torch.equal(y.view(torch.int16), y2.view(torch.int16))


def test_ln_glm_square_config(ops, orc):
    wl = W.glm_square()
    t = wl.tensors
    run_ln(ops, orc, t["x"].to(DEV), t["scale"].to(DEV), t["shift"].to(DEV), wl.meta["eps"], what="(1,4096,4096)")


@pytest.mark.parametrize("D", [4, 8, 12, 60, 64, 520, 1000, 2240, 3072, 4096, 4100, 8192, 12288, 16384,
                               16392, 20000, 32768, 65536])
def test_ln_hidden_sizes(ops, orc, D):
    g = torch.Generator().manual_seed(D)
    B, S = 3, 5
    x = rand_bf16((B, S, D), g, std=3.0, mean=0.5).to(DEV)
    sc = rand_bf16((B, D), g, std=0.1).to(DEV)
    sh = rand_bf16((B, D), g, std=0.1).to(DEV)
    run_ln(ops, orc, x, sc, sh, 1e-6, what="D=%d" % D)


def test_ln_long_rows_last_round(ops, orc):
    """16-wave blocks of 4 rows of 16384 elements would run one full round and an eighth of
    another: one row per block instead (same lanes and merges)."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    S = 4 * (cus + cus // 8)
    g = torch.Generator().manual_seed(S)
    x = rand_bf16((1, S, 16384), g, std=2.0).to(DEV)
    sc = rand_bf16((1, 16384), g, std=0.1).to(DEV)
    sh = rand_bf16((1, 16384), g, std=0.1).to(DEV)
    run_ln(ops, orc, x, sc, sh, 1e-6, check_fp64=False, what="(1,%d,16384)" % S)


# rows of 7-8 full vector steps (D = 3584, 4096) take 16-wave blocks; with too few rows to fill
# half the compute units that way they take the row kernel (same lanes and merges)
@pytest.mark.parametrize("D", [3584, 4096])
@pytest.mark.parametrize("B,S", [(1, 64), (2, 300), (1, 1024), (1, 2048)])
def test_ln_few_long_rows(ops, orc, D, B, S):
    g = torch.Generator().manual_seed(D + 7 * S + B)
    x = rand_bf16((B, S, D), g, std=2.0, mean=0.5).to(DEV)
    sc = rand_bf16((B, D), g, std=0.1).to(DEV)
    sh = rand_bf16((B, D), g, std=0.1).to(DEV)
    run_ln(ops, orc, x, sc, sh, 1e-6, check_fp64=False, what="few rows (%d,%d,%d)" % (B, S, D))


# more rows of 7-8 full steps than 16-wave blocks hold at one per wave: 4-wave blocks that
# prefetch the next row take them (same lanes and merges); ragged last blocks, several samples
@pytest.mark.parametrize("D,B,extra", [(4096, 1, 257), (3584, 2, 3), (4096, 3, 1000)])
def test_ln_many_long_rows(ops, orc, D, B, extra):
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    S = (16 * cus + extra + B - 1) // B
    g = torch.Generator().manual_seed(D + S + B)
    x = rand_bf16((B, S, D), g, std=2.0, mean=0.5).to(DEV)
    sc = rand_bf16((B, D), g, std=0.1).to(DEV)
    sh = rand_bf16((B, D), g, std=0.1).to(DEV)
    run_ln(ops, orc, x, sc, sh, 1e-6, check_fp64=False, what="many rows (%d,%d,%d)" % (B, S, D))


# rows with a partial last vector step whose instantiations hold fewer blocks per compute unit
# than their shape asks for: the launch is sized to what is held (same lanes and merges), so
# some waves walk two rows
@pytest.mark.parametrize("B,S,D", [(1, 5120, 2240), (1, 4096, 4000), (2, 2600, 1800), (3, 1800, 3000),
                                   (2, 2100, 3840)])
def test_ln_ragged_rows_held_blocks(ops, orc, B, S, D):
    g = torch.Generator().manual_seed(B * S + D)
    x = rand_bf16((B, S, D), g, std=2.0, mean=0.5).to(DEV)
    sc = rand_bf16((B, D), g, std=0.1).to(DEV)
    sh = rand_bf16((B, D), g, std=0.1).to(DEV)
    run_ln(ops, orc, x, sc, sh, 1e-6, check_fp64=False, what="held blocks (%d,%d,%d)" % (B, S, D))


# rows held by W = 1, 2, 4, 8, 16 waves (the cross-wave merge through LDS), with every lane
# full (D = 4096 W) or a ragged last step (and V = 4 when D % 8 != 0)
WAVE_ROWS = [(4096, 1), (4092, 1), (8192, 2), (4100, 2), (8200, 4), (16384, 4), (12296, 4), (32768, 8),
             (16392, 8), (32764, 8), (65536, 16), (40968, 16), (65532, 16)]


@pytest.mark.parametrize("D,W", WAVE_ROWS)
def test_ln_waves_per_row(ops, orc, D, W):
    """The order the library reports for the row (W waves, L = 64 W lanes) is the one the
    kernels follow, on contiguous rows, padded (strided) rows and misaligned rows."""
    from modulate_ln_amd import _native as N

    o = N.order_for(N.OP_LN_MODULATE, D)
    assert (o.W, o.L) == (W, 64 * W)
    g = torch.Generator().manual_seed(7 * D + W)
    B, S = 2, 3
    x = rand_bf16((B, S, D), g, std=2.0, mean=-1.0).to(DEV)
    sc = rand_bf16((B, D), g, std=0.1).to(DEV)
    sh = rand_bf16((B, D), g, std=0.1).to(DEV)
    run_ln(ops, orc, x, sc, sh, 1e-6, what="W=%d D=%d" % (W, D))
    big = rand_bf16((B, S, D + 24), g).to(DEV)
    run_ln(ops, orc, big[:, :, 8:8 + D], sc, sh, 1e-5, what="padded W=%d D=%d" % (W, D))
    run_ln(ops, orc, big[:, :, 1:1 + D], sc, sh, 1e-5, what="misaligned W=%d D=%d" % (W, D))


def shared_table_rows(W: int, B: int, half: bool = False) -> int:
    """Rows per sample that send rows of W = 2 or 4 waves to the shared-table kernel: blocks of
    16 / W rows of one sample, at least three quarters of the compute units' worth of them (in
    one round), and a partial last block in every sample.  half: 8-wave blocks of 8 / W rows
    instead (too few rows for 16-wave blocks to fill three quarters of the compute units, enough
    for 8-wave blocks to, in one round)."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    if half:
        P = 8 // W
        blocks = (4 * cus + 4) // 5  # 80 % of the compute units
        return P * ((blocks + B - 1) // B) - 1
    P = 16 // W
    blocks = (3 * cus + 3) // 4
    return P * ((blocks + B - 1) // B) + P // 2


# vector-aligned rows of 4097 .. 16384 elements, enough of them: a block of 16 waves holds 16 / W
# rows of one sample and builds the sample's tables once; the lanes and merges are those of one
# row per block, so the order (and the bits) stay the same.  Whole blocks, a partial last block
# per sample, several samples; fewer rows per sample (S given) take one row per block.
@pytest.mark.parametrize("D,W", [(8192, 2), (5120, 2), (8200, 4), (16384, 4), (12296, 4)])
@pytest.mark.parametrize("B,S", [(1, None), (2, None), (1, "half"), (3, 9)])
def test_ln_waves_per_row_shared_tables(ops, orc, D, W, B, S):
    from modulate_ln_amd import _native as N

    assert N.order_for(N.OP_LN_MODULATE, D).W == W
    S = shared_table_rows(W, B, half=True) if S == "half" else (S if S is not None else shared_table_rows(W, B))
    g = torch.Generator().manual_seed(11 * D + S)
    x = rand_bf16((B, S, D), g, std=2.0, mean=0.25).to(DEV)
    sc = rand_bf16((B, D), g, std=0.1).to(DEV)
    sh = rand_bf16((B, D), g, std=0.1).to(DEV)
    run_ln(ops, orc, x, sc, sh, 1e-6, what="shared tables W=%d D=%d (%d,%d)" % (W, D, B, S))


@pytest.mark.parametrize("D", [8, 64, 520, 1000, 2240, 3072, 4096, 4104, 8192])
@pytest.mark.parametrize("B,S", [(1, 8), (2, 40), (3, 1024)])
def test_ln_transposed_storage(ops, orc, B, S, D):
    """x stored [B, D, S] (tokens contiguous) and read through a transposed view, as the
    permuted DiT activations are: same bits as the logical values give contiguously."""
    g = torch.Generator().manual_seed(31 * D + S)
    xt = rand_bf16((B, D, S), g, std=2.0, mean=-0.25).to(DEV)
    x = xt.transpose(1, 2)
    emb = rand_bf16((B, 6, D), g, std=0.1).to(DEV)
    y = run_ln(ops, orc, x, emb[:, 5], emb[:, 0], 1e-6, what="transposed B=%d S=%d D=%d" % (B, S, D))
    y2 = ops.ln_modulate(x.contiguous(), emb[:, 5], emb[:, 0], 1e-6)
    assert torch.equal(y.view(torch.int16), y2.view(torch.int16))


@pytest.mark.parametrize("B,S", [(1, 1), (1, 37), (3, 1), (3, 37), (2, 1024)])
def test_ln_rows(ops, orc, B, S):
    g = torch.Generator().manual_seed(100 * B + S)
    D = 2240
    x = (rand_bf16((B, S, D), g) * 4).to(DEV)
    emb = rand_bf16((B, 2, D), g, std=0.1).to(DEV)
    run_ln(ops, orc, x, emb[:, 1], emb[:, 0], 1e-6, what="B=%d S=%d" % (B, S))


def test_ln_broadcast_single_adaln_row(ops, orc):
    g = torch.Generator().manual_seed(7)
    x = rand_bf16((3, 9, 512), g).to(DEV)
    sc = rand_bf16((1, 512), g, std=0.1).to(DEV)
    sh = rand_bf16((1, 512), g, std=0.1).to(DEV)
    run_ln(ops, orc, x, sc, sh, 1e-6, what="broadcast row")


def test_ln_inplace(ops, orc):
    g = torch.Generator().manual_seed(8)
    x = rand_bf16((2, 33, 4096), g).to(DEV)
    sc = rand_bf16((2, 4096), g, std=0.1).to(DEV)
    sh = rand_bf16((2, 4096), g, std=0.1).to(DEV)
    ref = ops.ln_modulate(x, sc, sh, 1e-5)
    x2 = x.clone()
    y = ops.ln_modulate(x2, sc, sh, 1e-5, out=x2)
    assert y.data_ptr() == x2.data_ptr()
    assert torch.equal(x2.view(torch.int16), ref.view(torch.int16))


@pytest.mark.parametrize("D", [512, 2240, 4100])
def test_ln_misaligned_and_strided(ops, orc, D):
    """Views that defeat the vector loads: odd element offsets, padded rows, a
    general stride on the hidden dim.  Same bits as the contiguous path."""
    g = torch.Generator().manual_seed(9 + D)
    B, S = 2, 7
    big = rand_bf16((B, S, D + 3), g).to(DEV)
    x = big[:, :, 1:D + 1]  # odd offset, row stride D+3
    emb = rand_bf16((B, 3 * D + 1), g, std=0.1).to(DEV)
    sc = emb[:, 1:D + 1]
    sh = emb[:, D + 1:2 * D + 1]
    run_ln(ops, orc, x, sc, sh, 1e-6, what="misaligned D=%d" % D)
    xs = rand_bf16((B, 2 * D, S), g).to(DEV)[:, ::2, :].transpose(1, 2)  # hidden stride 2*S, token stride 1
    run_ln(ops, orc, xs, sc, sh, 1e-6, what="strided D=%d" % D)


def test_ln_special_values(ops, orc):
    """Constant rows (out = +0), huge and tiny magnitudes, zero eps on a non-constant row."""
    D = 2240
    rows = [torch.full((D,), 3.5), torch.full((D,), -1000.0), torch.zeros(D),
            torch.linspace(-1e30, 1e30, D), torch.linspace(-1e-30, 1e-30, D)]
    x = torch.stack(rows)[None].to(torch.bfloat16)
    z = torch.zeros(1, D, dtype=torch.bfloat16)
    y = run_ln(ops, orc, x.to(DEV), z.to(DEV), z.to(DEV), 1e-6, check_fp64=False, what="special")
    assert torch.all(y[0, :3].view(torch.int16) == 0)
    x2 = torch.randn(1, 4, 512).to(torch.bfloat16)
    run_ln(ops, orc, x2.to(DEV), z[:, :512].to(DEV), z[:, :512].to(DEV), 0.0, what="eps=0")


def test_ln_nan_propagates(ops, orc):
    D = 512
    x = torch.randn(1, 3, D).to(torch.bfloat16)
    x[0, 1, 17] = float("nan")
    z = torch.zeros(1, D, dtype=torch.bfloat16)
    y = ops.ln_modulate(x.to(DEV), z.to(DEV), z.to(DEV), 1e-6).cpu()
    assert torch.isnan(y[0, 1]).all()
    assert not torch.isnan(y[0, 0]).any() and not torch.isnan(y[0, 2]).any()


def test_ln_empty(ops):
    x = torch.empty(0, 5, 512, dtype=torch.bfloat16, device=DEV)
    sc = torch.zeros(0, 512, dtype=torch.bfloat16, device=DEV)
    y = ops.ln_modulate(x, sc, sc, 1e-6)
    assert y.shape == (0, 5, 512)


def test_ln_rejects_bad_input(ops):
    x = torch.randn(1, 4, 6, device=DEV).to(torch.bfloat16)
    sc = torch.zeros(1, 6, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(ops.AdalnError):
        ops.ln_modulate(x, sc, sc, 1e-6)
    with pytest.raises(TypeError):
        ops.ln_modulate(x.float(), sc, sc, 1e-6)


def test_ln_vs_rocm_eager_tolerance(ops):
    """External sanity net (not bitwise): ROCm PyTorch's own eager chain, with its own
    reduction order, agrees within one bf16 ulp of the largest intermediate."""
    wl = W.glm_square(S=512)
    t = {k: v.to(DEV) for k, v in wl.tensors.items()}
    x, sc, sh = t["x"], t["scale"], t["shift"]
    eager = torch.nn.functional.layer_norm(x, (4096,), eps=1e-5) * (1 + sc[:, None]) + sh[:, None]
    ours = ops.ln_modulate(x, sc, sh, 1e-5)
    xh = torch.nn.functional.layer_norm(x.float(), (4096,), eps=1e-5)
    big = torch.maximum(torch.maximum((xh * (1 + sc[:, None].float())).abs(), sh[:, None].float().abs()),
                        ours.float().abs())
    assert torch.all((eager.float() - ours.float()).abs() <= big * 2.0 ** -7 + 1e-30)


# ---------------------------------------------------------------------------
# residual_gate_add
# ---------------------------------------------------------------------------

def run_rga(ops, orc, res, gate, upd, *, out=None, what=""):
    B, S, D = res.shape
    g2 = gate[:, 0] if gate.dim() == 3 else gate
    want = orc.residual_gate_add(bits(res.reshape(B * S, D) if res.is_contiguous() else res.contiguous().reshape(B * S, D)),
                                 bits(g2.expand(B, D)),
                                 bits(upd.contiguous().reshape(B * S, D)), S, FP32)
    y = ops.residual_gate_add(res, gate, upd, out=out)
    torch.cuda.synchronize()
    assert_bits_equal(bits(y.reshape(B * S, D)), want, "residual_gate_add " + what)
    return y


def test_rga_glm_square_config(ops, orc):
    wl = W.glm_square()
    t = wl.tensors
    x = t["x"].to(DEV)
    h = ops.ln_modulate(x, t["scale"].to(DEV), t["shift"].to(DEV), 1e-5)
    run_rga(ops, orc, x, t["gate"].to(DEV), h, what="(1,4096,4096) after ln_modulate")
    run_rga(ops, orc, x, t["gate"].to(DEV), t["update"].to(DEV), what="(1,4096,4096)")


@pytest.mark.parametrize("D", [1, 3, 4, 7, 8, 12, 520, 2240, 4096, 4100, 12288])
def test_rga_hidden_sizes(ops, orc, D):
    g = torch.Generator().manual_seed(500 + D)
    B, S = 2, 9
    res = rand_bf16((B, S, D), g).to(DEV)
    upd = rand_bf16((B, S, D), g, std=4.0).to(DEV)
    gate = rand_bf16((B, D), g, std=0.1).to(DEV)
    run_rga(ops, orc, res, gate, upd, what="D=%d" % D)


def test_rga_large_one_shot_ragged(ops, orc):
    # 2*4100*4104 elements (>= 2^25: the one-shot grid), 513 vectors per row
    # (a ragged last block), then the same update in place
    g = torch.Generator().manual_seed(57)
    B, S, D = 2, 4100, 4104
    res = rand_bf16((B, S, D), g).to(DEV)
    upd = rand_bf16((B, S, D), g, std=4.0).to(DEV)
    gate = rand_bf16((B, D), g, std=0.1).to(DEV)
    ref = run_rga(ops, orc, res, gate, upd, what="(2,4100,4104)")
    ops.residual_gate_add(res, gate, upd, out=res)
    torch.cuda.synchronize()
    assert torch.equal(res.view(torch.int16), ref.view(torch.int16))


def device_normal_bf16(shape, seed, std=1.0):
    """A large seeded normal tensor drawn on the device (the host draw of billions of values
    would take minutes); the oracle gets the same values back through a copy."""
    g = torch.Generator(device=DEV).manual_seed(seed)
    return (torch.randn(shape, generator=g, device=DEV) * std).to(torch.bfloat16)


def test_rga_row_beyond_2g_elements(ops, orc):
    """One row of 2^31 + 4096 elements (4 GiB per tensor): the one-shot grid's element offsets
    pass 2^31, so its indexing must be 64-bit.  The oracle checks the first and the last 8192
    elements (the op is element-wise with a per-sample gate)."""
    D = (1 << 31) + 4096
    res = device_normal_bf16((1, 1, D), 1)
    upd = device_normal_bf16((1, 1, D), 2)
    gate = device_normal_bf16((1, D), 3, std=0.5)
    y = ops.residual_gate_add(res, gate, upd)
    torch.cuda.synchronize()
    for lo in (0, D - 8192):
        sl = slice(lo, lo + 8192)
        want = orc.residual_gate_add(bits(res[0, :, sl]), bits(gate[:, sl]), bits(upd[0, :, sl]), 1, FP32)
        assert_bits_equal(bits(y[0, :, sl]), want, "rga beyond 2^31 at %d" % lo)
    del res, upd, gate, y
    torch.cuda.empty_cache()


def test_rga_inplace_and_views(ops, orc):
    g = torch.Generator().manual_seed(11)
    B, S, D = 2, 17, 3072
    res = rand_bf16((B, S, D), g).to(DEV)
    upd = rand_bf16((B, S, D), g).to(DEV)
    emb = rand_bf16((B, 6, D), g, std=0.1).to(DEV)
    gate = emb[:, 2]
    ref = run_rga(ops, orc, res, gate, upd)
    r2 = res.clone()
    ops.residual_gate_add(r2, gate, upd, out=r2)
    assert torch.equal(r2.view(torch.int16), ref.view(torch.int16))
    u2 = upd.clone()
    ops.residual_gate_add(res, gate, u2, out=u2)
    assert torch.equal(u2.view(torch.int16), ref.view(torch.int16))
    # strided residual (padded rows) and misaligned update
    bigr = rand_bf16((B, S, D + 8), g).to(DEV)
    bigu = rand_bf16((B, S, D + 1), g).to(DEV)
    run_rga(ops, orc, bigr[:, :, :D], gate, bigu[:, :, 1:], what="views")
    # signed zeros: residual -0, gate 0, update >= 0 -> +0
    rz = torch.full((1, 1, 8), -0.0, dtype=torch.bfloat16, device=DEV)
    y = ops.residual_gate_add(rz, torch.zeros(1, 8, dtype=torch.bfloat16, device=DEV),
                              torch.ones(1, 1, 8, dtype=torch.bfloat16, device=DEV))
    assert torch.all(y.view(torch.int16) == 0)


# ---------------------------------------------------------------------------
# qk_head_layernorm
# ---------------------------------------------------------------------------

def run_qk(ops, orc, q, k, w, eps, *, what="", q_out=None, k_out=None):
    B, S, H, Dh = q.shape
    V, L = order(N_OP_QK, Dh, q)
    assert order(N_OP_QK, Dh, k) == (V, L)
    wq, bq, wk, bk = w if w is not None else (None, None, None, None)
    qo, ko = ops.qk_head_layernorm(q, k, wq, bq, wk, bk, eps, q_out=q_out, k_out=k_out)
    torch.cuda.synchronize()
    for name, src, o, ww, bb in (("q", q, qo, wq, bq), ("k", k, ko, wk, bk)):
        want = orc.qk_head_layernorm(bits(src.contiguous().reshape(-1, Dh)), bits(ww) if ww is not None else None,
                                     bits(bb) if bb is not None else None, eps, FP32, V=V, L=L)
        assert_bits_equal(bits(o.reshape(-1, Dh)), want, "qk %s %s" % (name, what))
    return qo, ko


def test_qk_glm_config(ops, orc):
    wl = W.glm_qk()
    t = {k: v.to(DEV) for k, v in wl.tensors.items()}
    run_qk(ops, orc, t["q"], t["k"], (t["wq"], t["bq"], t["wk"], t["bk"]), wl.meta["eps"], what="(1,4360,32,128)")


@pytest.mark.parametrize("Dh", [4, 12, 64, 96, 128, 132, 256])
@pytest.mark.parametrize("affine", [True, False])
def test_qk_head_sizes(ops, orc, Dh, affine):
    g = torch.Generator().manual_seed(Dh)
    B, S, H = 2, 5, 3
    q = rand_bf16((B, S, H, Dh), g).to(DEV)
    k = rand_bf16((B, S, H, Dh), g, std=2.0).to(DEV)
    w = tuple(rand_bf16((Dh,), g, mean=m, std=s).to(DEV) for m, s in ((1, .05), (0, .02), (1, .05), (0, .02)))
    run_qk(ops, orc, q, k, w if affine else None, 1e-6, what="Dh=%d affine=%s" % (Dh, affine))


def test_qk_packed_qkv_views_and_inplace(ops, orc):
    """q and k read straight out of a packed [B,S,3,H,Dh] projection (non-uniform row
    strides), and in-place on contiguous inputs."""
    g = torch.Generator().manual_seed(21)
    B, S, H, Dh = 2, 6, 4, 128
    qkv = rand_bf16((B, S, 3, H, Dh), g).to(DEV)
    q, k = qkv[:, :, 0], qkv[:, :, 1]
    w = tuple(rand_bf16((Dh,), g, mean=m, std=.05).to(DEV) for m in (1, 0, 1, 0))
    qo, ko = run_qk(ops, orc, q, k, w, 1e-6, what="packed qkv")
    q2, k2 = q.contiguous(), k.contiguous()
    ops.qk_head_layernorm(q2, k2, *w, 1e-6, q_out=q2, k_out=k2)
    assert torch.equal(q2.view(torch.int16), qo.view(torch.int16))
    assert torch.equal(k2.view(torch.int16), ko.view(torch.int16))


# ---------------------------------------------------------------------------
# bias + tanh-GELU
# ---------------------------------------------------------------------------

def bf16_ulp(v: np.ndarray) -> np.ndarray:
    a = np.abs(v).astype(np.float64)
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -126)))
    return 2.0 ** (e - 7)


def check_gelu(ops, orc, x, bias, what=""):
    y = ops.bias_gelu_tanh(x, bias)
    torch.cuda.synchronize()
    want, val = orc.bias_gelu_tanh(bits(x.contiguous()), bits(bias))
    got = f32(bits(y)).astype(np.float64)
    ref = f32(want).astype(np.float64)
    diff = np.abs(got - ref)
    assert np.all(diff <= bf16_ulp(val) + 2.0 ** -133), what
    assert np.mean(got == ref) > 0.99, what


def test_gelu_wan_config_sampled_rows(ops, orc):
    wl = W.wan_bias_gelu()
    x = wl.tensors["x"].to(DEV)
    bias = wl.tensors["bias"].to(DEV)
    y = ops.bias_gelu_tanh(x, bias)
    torch.cuda.synchronize()
    rows = torch.linspace(0, x.shape[0] - 1, 4096).long()  # a quarter of the rows, first and last included
    want, val = orc.bias_gelu_tanh(bits(wl.tensors["x"][rows]), bits(wl.tensors["bias"]))
    got = f32(bits(y[rows.to(DEV)])).astype(np.float64)
    ref = f32(want).astype(np.float64)
    assert np.all(np.abs(got - ref) <= bf16_ulp(val) + 2.0 ** -133)
    assert np.mean(got == ref) > 0.99


@pytest.mark.parametrize("width", [1, 3, 4, 8, 100, 12288])
def test_gelu_widths(ops, orc, width):
    g = torch.Generator().manual_seed(width)
    x = rand_bf16((7, width), g, std=3.0).to(DEV)
    bias = rand_bf16((width,), g, std=0.5).to(DEV)
    check_gelu(ops, orc, x, bias, "width=%d" % width)


def test_gelu_every_bf16_value(ops, orc):
    """All 65536 bf16 patterns as z (bias 0): finite results within one bf16 ulp of the fp64
    oracle, and the non-finite cases as the oracle has them (NaN in, NaN out; +inf -> +inf;
    -inf -> NaN, the eager formula's -inf * 0)."""
    z = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    x = torch.from_numpy(z.view(np.int16).copy()).view(torch.bfloat16)[None].to(DEV)
    zero = torch.zeros(x.shape[1], dtype=torch.bfloat16, device=DEV)
    y = ops.bias_gelu_tanh(x, zero)
    torch.cuda.synchronize()
    want, val = orc.bias_gelu_tanh(z[None], bits(zero))
    got = f32(bits(y)).astype(np.float64)[0]
    ref = f32(want).astype(np.float64)[0]
    fin = np.isfinite(ref)
    diff = np.abs(got[fin] - ref[fin])
    assert np.all(diff <= bf16_ulp(val[0][fin]) + 2.0 ** -133)
    assert np.mean(got[fin] == ref[fin]) > 0.99
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    inf = np.isinf(ref)
    assert np.array_equal(got[inf], ref[inf])


def test_gelu_tails_and_views(ops, orc):
    z = torch.cat([torch.linspace(-15, 15, 4096), torch.tensor([0.0, -0.0, 1e-30, -1e-30, 88.0, -88.0])])
    x = z.to(torch.bfloat16)[None].to(DEV)
    zero = torch.zeros(x.shape[1], dtype=torch.bfloat16, device=DEV)
    check_gelu(ops, orc, x, zero, "tails")
    g = torch.Generator().manual_seed(5)
    big = rand_bf16((5, 1030), g).to(DEV)
    check_gelu(ops, orc, big[:, 3:1027], rand_bf16((1024,), g, std=0.1).to(DEV), "strided")


# ---------------------------------------------------------------------------
# the 20-block DiT chain
# ---------------------------------------------------------------------------

def oracle_chain_rows(orc, x_rows, embs, b, eps):
    """Oracle chain on a few rows of batch sample b (rows are independent)."""
    D = x_rows.shape[1]
    V, L = order(N_OP_LN, D)
    x = x_rows
    S = x.shape[0]
    for emb in embs:
        e = bits(emb[b])  # [6, D]
        for j in (0, 3):
            sh, sc, gt = e[j:j + 1], e[j + 1:j + 2], e[j + 2:j + 3]
            h, _, _ = orc.ln_modulate(x, sc, sh, S, eps, FP32, V=V, L=L)
            x = orc.residual_gate_add(x, gt, h, S, FP32)
    return x


def gpu_chain(ops, x, embs_dev, eps):
    h = torch.empty_like(x)
    for emb in embs_dev:
        for j in (0, 3):
            ops.ln_modulate(x, emb[:, j + 1], emb[:, j], eps, out=h)
            ops.residual_gate_add(x, emb[:, j + 2], h, out=x)
    return x


def oracle_chain(orc, x0, embs, eps):
    """The oracle's 20-block chain on every row of x0 [B, S, D] (per-sample adaLN rows)."""
    B, S, D = x0.shape
    V, L = order(N_OP_LN, D)
    x = bits(x0.reshape(B * S, D))
    for emb in embs:
        e = bits(emb)  # [B, 6, D]
        for j in (0, 3):
            sh, sc, gt = e[:, j], e[:, j + 1], e[:, j + 2]
            h, _, _ = orc.ln_modulate(x, sc, sh, S, eps, FP32, V=V, L=L)
            x = orc.residual_gate_add(x, gt, h, S, FP32)
    return x


def test_dit_chain_config_every_row(ops, orc):
    """The 20-block chain on (4,4096,3072): every one of the 16384 rows bit-exact against the
    oracle's chain (80 kernel launches against 80 oracle calls)."""
    wl = W.dit_chain()
    x0 = wl.tensors["x"]
    embs = wl.tensors["embs"]
    x = gpu_chain(ops, x0.to(DEV).clone(), [e.to(DEV) for e in embs], wl.meta["eps"])
    torch.cuda.synchronize()
    B, S, D = x0.shape
    want = oracle_chain(orc, x0, embs, wl.meta["eps"])
    assert_bits_equal(bits(x.reshape(B * S, D)), want, "chain (4,4096,3072)")
