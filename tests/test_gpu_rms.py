"""Parity of the RMSNorm kernels -- rmsnorm_scale_shift and qk_rmsnorm -- with
the CPU oracle, through the C ABI.

Bar: bit-exact against the oracle's fixed-order fp32 mode, run in the order
the library reports (adaln_order_for: V elements per vector, L = 64 W lanes
per row, 16 per head); the fp32 1/rms of each row within 1e-5 relative of
the fp64 two-pass mode.  Same shapes and layouts as the LayerNorm tests:
every kernel family (tabled rows, transposed tiles, general rows, rows of
several waves; heads in flight, general heads).
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

from modulate_ln_amd import workloads as W

from test_gpu_parity import DEV, FP32, N_OP_QK_RMS, N_OP_RMS, FP64, assert_bits_equal, bits, order, rand_bf16

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ops():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import modulate_ln_amd as m

    m._native.lib()
    return m


def run_rms(ops, orc, x_dev, scale_dev, shift_dev, eps, *, out=None, check_fp64=True, what=""):
    B, S, D = x_dev.shape
    rinv = torch.empty(B * S, dtype=torch.float32, device=DEV)
    x_log = bits(x_dev.contiguous().reshape(B * S, D))
    sc = scale_dev[:, 0] if scale_dev.dim() == 3 else scale_dev
    sh = shift_dev[:, 0] if shift_dev.dim() == 3 else shift_dev
    sc_b, sh_b = bits(sc.expand(B, D)), bits(sh.expand(B, D))
    y = ops.rmsnorm_scale_shift(x_dev, scale_dev, shift_dev, eps, out=out, rinv_out=rinv)
    torch.cuda.synchronize()
    V, L = order(N_OP_RMS, D, x_dev)
    want, r32 = orc.rmsnorm_scale_shift(x_log, sc_b, sh_b, S, eps, FP32, V=V, L=L)
    assert_bits_equal(bits(y.reshape(B * S, D)), want, "rmsnorm_scale_shift %s" % what)
    assert np.array_equal(rinv.cpu().numpy().astype(np.float64), r32), "rinv " + what
    if check_fp64:
        _, r64 = orc.rmsnorm_scale_shift(x_log, sc_b, sh_b, S, eps, FP64)
        assert np.all(np.abs(r32 - r64) <= 1e-5 * r64), what
    return y


def test_rms_glm_square_shape(ops, orc):
    wl = W.glm_square()
    t = wl.tensors
    run_rms(ops, orc, t["x"].to(DEV), t["scale"].to(DEV), t["shift"].to(DEV), wl.meta["eps"], what="(1,4096,4096)")


def test_rms_small_and_sana_transposed_shapes(ops, orc):
    wl = W.ln_small()
    t = wl.tensors
    run_rms(ops, orc, t["x"].to(DEV), t["scale"].to(DEV), t["shift"].to(DEV), wl.meta["eps"], what="(1,256,512)")
    wl = W.sana_transposed()
    xt = wl.tensors["xt"].to(DEV)
    emb = wl.tensors["emb"].to(DEV)
    y = run_rms(ops, orc, xt.transpose(1, 2), emb[:, 5], emb[:, 0], wl.meta["eps"], what="sana transposed")
    y2 = ops.rmsnorm_scale_shift(xt.transpose(1, 2).contiguous(), emb[:, 5], emb[:, 0], wl.meta["eps"])
    assert torch.equal(y.view(torch.int16), y2.view(torch.int16))


@pytest.mark.parametrize("D", [4, 8, 12, 60, 64, 520, 1000, 2240, 3072, 4096, 4100, 8192, 12288, 16384,
                               16392, 20000, 65536])
def test_rms_hidden_sizes(ops, orc, D):
    g = torch.Generator().manual_seed(900 + D)
    B, S = 3, 5
    x = rand_bf16((B, S, D), g, std=3.0, mean=0.5).to(DEV)
    sc = rand_bf16((B, D), g, std=0.1).to(DEV)
    sh = rand_bf16((B, D), g, std=0.1).to(DEV)
    run_rms(ops, orc, x, sc, sh, 1e-6, what="D=%d" % D)


@pytest.mark.parametrize("S,D", [(4096, 4000), (4096, 3840), (5120, 2240)])
def test_rms_ragged_rows_held_blocks(ops, orc, S, D):
    """Rows with a partial last step, enough of them for one row per wave of the launch: their
    instantiations read each step's table values at that step (no look-ahead), so the waves the
    launch asks for fit."""
    g = torch.Generator().manual_seed(S + D)
    x = rand_bf16((1, S, D), g, std=2.0, mean=0.5).to(DEV)
    sc = rand_bf16((1, D), g, std=0.1).to(DEV)
    sh = rand_bf16((1, D), g, std=0.1).to(DEV)
    run_rms(ops, orc, x, sc, sh, 1e-6, check_fp64=False, what="held blocks (1,%d,%d)" % (S, D))


@pytest.mark.parametrize("D,W", [(8192, 2), (16384, 4)])
def test_rms_long_rows_shared_tables(ops, orc, D, W):
    """Rows of 2 and 4 waves, enough per sample that blocks of 16 waves hold 8 or 4 rows of a
    sample and share its tables (a partial last block per sample)."""
    from test_gpu_parity import shared_table_rows

    S = shared_table_rows(W, 2)
    g = torch.Generator().manual_seed(950 + D)
    x = rand_bf16((2, S, D), g, std=3.0, mean=0.5).to(DEV)
    sc = rand_bf16((2, D), g, std=0.1).to(DEV)
    sh = rand_bf16((2, D), g, std=0.1).to(DEV)
    run_rms(ops, orc, x, sc, sh, 1e-6, what="shared tables D=%d" % D)


@pytest.mark.parametrize("D", [8, 520, 2240, 4096, 4104])
@pytest.mark.parametrize("B,S", [(1, 8), (3, 1024)])
def test_rms_transposed_storage(ops, orc, B, S, D):
    g = torch.Generator().manual_seed(37 * D + S)
    xt = rand_bf16((B, D, S), g, std=2.0, mean=-0.25).to(DEV)
    emb = rand_bf16((B, 6, D), g, std=0.1).to(DEV)
    run_rms(ops, orc, xt.transpose(1, 2), emb[:, 5], emb[:, 0], 1e-6, what="transposed B=%d S=%d D=%d" % (B, S, D))


@pytest.mark.parametrize("B,S", [(1, 1), (3, 37), (2, 1024)])
def test_rms_rows_views_inplace(ops, orc, B, S):
    g = torch.Generator().manual_seed(200 * B + S)
    D = 2240
    x = (rand_bf16((B, S, D), g) * 4).to(DEV)
    emb = rand_bf16((B, 2, D), g, std=0.1).to(DEV)
    ref = run_rms(ops, orc, x, emb[:, 1], emb[:, 0], 1e-6, what="B=%d S=%d" % (B, S))
    x2 = x.clone()
    ops.rmsnorm_scale_shift(x2, emb[:, 1], emb[:, 0], 1e-6, out=x2)
    assert torch.equal(x2.view(torch.int16), ref.view(torch.int16))
    big = rand_bf16((B, S, D + 3), g).to(DEV)
    run_rms(ops, orc, big[:, :, 1:D + 1], emb[:, 1], emb[:, 0], 1e-6, what="misaligned B=%d S=%d" % (B, S))


def test_rms_special_values(ops, orc):
    """Constant rows normalize to +-1 (c != 0) and +0 (c = 0); NaN poisons only its row;
    eps = 0 on a non-zero row."""
    D = 2240
    rows = [torch.full((D,), 3.5), torch.full((D,), -1000.0), torch.zeros(D),
            torch.linspace(-1e30, 1e30, D), torch.linspace(-1e-30, 1e-30, D)]
    x = torch.stack(rows)[None].to(torch.bfloat16)
    z = torch.zeros(1, D, dtype=torch.bfloat16)
    y = run_rms(ops, orc, x.to(DEV), z.to(DEV), z.to(DEV), 1e-6, check_fp64=False, what="special")
    assert torch.all(y[0, 0] == 1.0) and torch.all(y[0, 1] == -1.0)
    assert torch.all(y[0, 2].view(torch.int16) == 0)
    x2 = torch.randn(1, 4, 512).to(torch.bfloat16)
    run_rms(ops, orc, x2.to(DEV), z[:, :512].to(DEV), z[:, :512].to(DEV), 0.0, what="eps=0")
    x2[0, 1, 17] = float("nan")
    y = ops.rmsnorm_scale_shift(x2.to(DEV), z[:, :512].to(DEV), z[:, :512].to(DEV), 1e-6).cpu()
    assert torch.isnan(y[0, 1]).all() and not torch.isnan(y[0, 0]).any()


def test_rms_vs_rocm_eager_tolerance(ops):
    """External sanity net (not bitwise): ROCm PyTorch's eager rms_norm, with its own reduction
    order and reciprocal square root.  x_hat (scale = shift = 0) agrees within one bf16 ulp; a
    one-ulp difference in x_hat moves y = bf16(x_hat * (1 + scale)) by at most 2^-7 of |x_hat *
    (1 + scale)| plus two half-ulp roundings, and out = bf16(y + shift) by one more half-ulp on
    each side, so the chain agrees within 3 * 2^-7 of its largest intermediate."""
    wl = W.glm_square(S=512)
    t = {k: v.to(DEV) for k, v in wl.tensors.items()}
    x, sc, sh = t["x"], t["scale"], t["shift"]
    z = torch.zeros_like(sc)
    xh_eager = torch.nn.functional.rms_norm(x, (4096,), eps=1e-5).float()
    xh_ours = ops.rmsnorm_scale_shift(x, z, z, 1e-5).float()
    assert torch.all((xh_eager - xh_ours).abs() <= xh_ours.abs() * 2.0 ** -7 + 1e-30)
    eager = torch.nn.functional.rms_norm(x, (4096,), eps=1e-5) * (1 + sc[:, None]) + sh[:, None]
    ours = ops.rmsnorm_scale_shift(x, sc, sh, 1e-5)
    xh = torch.nn.functional.rms_norm(x.float(), (4096,), eps=1e-5)
    big = torch.maximum(torch.maximum((xh * (1 + sc[:, None].float())).abs(), sh[:, None].float().abs()),
                        ours.float().abs())
    assert torch.all((eager.float() - ours.float()).abs() <= big * 3 * 2.0 ** -7 + 1e-30)


# ---------------------------------------------------------------------------
# qk_rmsnorm
# ---------------------------------------------------------------------------

def run_qk_rms(ops, orc, q, k, w, eps, *, what="", q_out=None, k_out=None):
    B, S, H, Dh = q.shape
    V, L = order(N_OP_QK_RMS, Dh, q)
    assert order(N_OP_QK_RMS, Dh, k) == (V, L)
    wq, wk = w if w is not None else (None, None)
    qo, ko = ops.qk_rmsnorm(q, k, wq, wk, eps, q_out=q_out, k_out=k_out)
    torch.cuda.synchronize()
    for name, src, o, ww in (("q", q, qo, wq), ("k", k, ko, wk)):
        want = orc.qk_rmsnorm(bits(src.contiguous().reshape(-1, Dh)), bits(ww) if ww is not None else None, eps,
                              FP32, V=V, L=L)
        assert_bits_equal(bits(o.reshape(-1, Dh)), want, "qk_rmsnorm %s %s" % (name, what))
    return qo, ko


def test_qk_rms_glm_shape(ops, orc):
    """(1,4360,32,128) q and k with weights ~N(1, 0.05) (the q/k LayerNorm shape)."""
    wl = W.glm_qk()
    t = {k: v.to(DEV) for k, v in wl.tensors.items()}
    run_qk_rms(ops, orc, t["q"], t["k"], (t["wq"], t["wk"]), wl.meta["eps"], what="(1,4360,32,128)")


@pytest.mark.parametrize("Dh", [4, 12, 64, 96, 128, 132, 256])
@pytest.mark.parametrize("weighted", [True, False])
def test_qk_rms_head_sizes(ops, orc, Dh, weighted):
    g = torch.Generator().manual_seed(3000 + Dh)
    B, S, H = 2, 5, 3
    q = rand_bf16((B, S, H, Dh), g).to(DEV)
    k = rand_bf16((B, S, H, Dh), g, std=2.0).to(DEV)
    w = tuple(rand_bf16((Dh,), g, mean=1.0, std=0.05).to(DEV) for _ in range(2))
    run_qk_rms(ops, orc, q, k, w if weighted else None, 1e-6, what="Dh=%d weighted=%s" % (Dh, weighted))


def test_qk_rms_packed_qkv_views_and_inplace(ops, orc):
    g = torch.Generator().manual_seed(41)
    B, S, H, Dh = 2, 6, 4, 128
    qkv = rand_bf16((B, S, 3, H, Dh), g).to(DEV)
    q, k = qkv[:, :, 0], qkv[:, :, 1]
    w = tuple(rand_bf16((Dh,), g, mean=1.0, std=.05).to(DEV) for _ in range(2))
    qo, ko = run_qk_rms(ops, orc, q, k, w, 1e-6, what="packed qkv")
    q2, k2 = q.contiguous(), k.contiguous()
    ops.qk_rmsnorm(q2, k2, *w, 1e-6, q_out=q2, k_out=k2)
    assert torch.equal(q2.view(torch.int16), qo.view(torch.int16))
    assert torch.equal(k2.view(torch.int16), ko.view(torch.int16))
    big = rand_bf16((B, S, H, Dh + 1), g).to(DEV)  # misaligned heads: the general kernel
    run_qk_rms(ops, orc, big[..., 1:], k, w, 1e-6, what="misaligned q")


def test_qk_rms_vs_rocm_eager_tolerance(ops):
    g = torch.Generator().manual_seed(43)
    q = rand_bf16((1, 64, 8, 128), g).to(DEV)
    w = rand_bf16((128,), g, mean=1.0, std=0.05).to(DEV)
    qo, _ = ops.qk_rmsnorm(q, q.clone(), w, w, 1e-6)
    eager = torch.nn.functional.rms_norm(q, (128,), weight=w, eps=1e-6)
    ref = torch.nn.functional.rms_norm(q.float(), (128,), weight=w.float(), eps=1e-6)
    assert torch.all((eager.float() - qo.float()).abs() <= ref.abs() * 2.0 ** -7 + 1e-30)
