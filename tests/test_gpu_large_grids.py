"""Shapes whose one-shot grids would count more work-items than a dispatch holds (2^32):
millions of samples of short rows, tens of millions of transposed tokens, hundreds of millions of
q/k heads.  The library keeps every launch under that count -- the row kernels, whose grids are
capped and walk the rows, take the largest shapes, and the q/k head kernel walks its heads with a
capped grid -- so every row is written.  Sampled rows, always including the last ones, are
bit-exact against the oracle in the order the library reports.

The inputs are seeded normal draws made on the device (a few GB each, too large to draw on the
host in a test); the oracle gets the sampled rows' input bits copied back from those tensors.
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

from test_gpu_parity import DEV, FP32, N_OP_FUSED, N_OP_LN, N_OP_QK, assert_bits_equal, bits, device_normal_bf16, order

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ops():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import modulate_ln_amd as m

    m._native.lib()  # fail loudly if the library is missing
    return m


def normal_dev(shape, seed, std=1.0, mean=0.0):
    t = device_normal_bf16(shape, seed, std)
    return t if mean == 0.0 else (t.float() + mean).to(torch.bfloat16)


def sample_rows(R: int, seed: int) -> torch.Tensor:
    """The first 256 rows, 1024 drawn from the rest, and the last 1024."""
    g = np.random.default_rng(seed)
    mid = g.integers(256, R - 1024, size=1024)
    idx = np.unique(np.concatenate([np.arange(256), mid, np.arange(R - 1024, R)]))
    return torch.from_numpy(idx).to(DEV)


def test_ln_modulate_many_samples(ops, orc):
    """(2^24 + 3, 1, 8) with per-sample adaLN rows: a block per sample would be 2^32 + 768
    work-items; the row kernel takes it."""
    B, S, D = (1 << 24) + 3, 1, 8
    x = normal_dev((B, S, D), 1)
    scale = normal_dev((B, D), 2, std=0.1)
    shift = normal_dev((B, D), 3, std=0.1)
    mean = torch.empty(B * S, dtype=torch.float32, device=DEV)
    rstd = torch.empty(B * S, dtype=torch.float32, device=DEV)
    y = ops.ln_modulate(x, scale, shift, 1e-6, mean_out=mean, rstd_out=rstd)
    torch.cuda.synchronize()
    idx = sample_rows(B, 4)
    V, L = order(N_OP_LN, D, x)
    want, m32, r32 = orc.ln_modulate(bits(x[idx, 0]), bits(scale[idx]), bits(shift[idx]), 1, 1e-6, FP32, V=V, L=L)
    assert_bits_equal(bits(y[idx, 0]), want, "ln_modulate (2^24+3,1,8)")
    assert np.array_equal(mean[idx].cpu().numpy().astype(np.float64), m32)
    assert np.array_equal(rstd[idx].cpu().numpy().astype(np.float64), r32)


def test_ln_modulate_long_transposed_run(ops, orc):
    """x stored [1, 8, 2^26] (transposed): 2^23 tiles of 8 tokens would be 2^32 work-items;
    the gathering row kernel takes it."""
    S, D = 1 << 26, 8
    xt = normal_dev((1, D, S), 5)
    x = xt.transpose(1, 2)  # [1, S, D], token stride 1
    scale = normal_dev((1, D), 6, std=0.1)
    shift = normal_dev((1, D), 7, std=0.1)
    rstd = torch.empty(S, dtype=torch.float32, device=DEV)
    y = ops.ln_modulate(x, scale, shift, 1e-6, rstd_out=rstd)
    torch.cuda.synchronize()
    del xt
    idx = sample_rows(S, 8)
    V, L = order(N_OP_LN, D, x)
    n = idx.numel()  # the sampled tokens as one sample of n rows
    want, _, r32 = orc.ln_modulate(bits(x[0, idx]), bits(scale), bits(shift), n, 1e-6, FP32, V=V, L=L)
    assert_bits_equal(bits(y[0, idx]), want, "ln_modulate transposed (1,2^26,8)")
    assert np.array_equal(rstd[idx].cpu().numpy().astype(np.float64), r32)


def test_residual_gate_add_ln_modulate_many_samples(ops, orc):
    """The fused update at (2^24 + 3, 1, 8): the unfused pair takes it, same bits."""
    B, S, D = (1 << 24) + 3, 1, 8
    res = normal_dev((B, S, D), 11)
    upd = normal_dev((B, S, D), 12)
    gate = normal_dev((B, D), 13, std=0.1)
    scale = normal_dev((B, D), 14, std=0.1)
    shift = normal_dev((B, D), 15, std=0.1)
    r_out, out = ops.residual_gate_add_ln_modulate(res, gate, upd, scale, shift, 1e-6)
    torch.cuda.synchronize()
    idx = sample_rows(B, 16)
    V, L = order(N_OP_FUSED, D, res)
    want_r, want, _, _ = orc.residual_gate_add_ln_modulate(bits(res[idx, 0]), bits(gate[idx]), bits(upd[idx, 0]),
                                                           bits(scale[idx]), bits(shift[idx]), 1, 1e-6, FP32,
                                                           V=V, L=L)
    assert_bits_equal(bits(r_out[idx, 0]), want_r, "fused residual (2^24+3,1,8)")
    assert_bits_equal(bits(out[idx, 0]), want, "fused out (2^24+3,1,8)")


def test_qk_head_layernorm_grid_walks_heads(ops, orc):
    """(1, 2^22 + 3, 64, 4) q and k: 2^28 + 192 heads per side, more than the head kernel's
    capped grid covers in one pass (2^23 blocks of 32 heads), so its groups walk the rest."""
    B, S, H, Dh = 1, (1 << 22) + 3, 64, 4
    q = normal_dev((B, S, H, Dh), 21)
    k = normal_dev((B, S, H, Dh), 22, std=2.0)
    w = tuple(normal_dev((Dh,), 23 + i, mean=m, std=s) for i, (m, s) in enumerate(((1, .05), (0, .02), (1, .05),
                                                                                    (0, .02))))
    qo, ko = ops.qk_head_layernorm(q, k, *w, 1e-6)
    torch.cuda.synchronize()
    R = B * S * H
    idx = sample_rows(R, 27)
    V, L = order(N_OP_QK, Dh, q)
    for name, src, o, ww, bb in (("q", q, qo, w[0], w[1]), ("k", k, ko, w[2], w[3])):
        want = orc.qk_head_layernorm(bits(src.reshape(R, Dh)[idx]), bits(ww), bits(bb), 1e-6, FP32, V=V, L=L)
        assert_bits_equal(bits(o.reshape(R, Dh)[idx]), want, "qk %s (1,2^22+3,64,4)" % name)
