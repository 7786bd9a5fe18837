"""One call of an entry point is one kernel dispatch: the device kernels the torch profiler records
around a prepared call (inputs and outputs made beforehand, so nothing else runs) are exactly
one, and it is one of this library's kernels."""

from __future__ import annotations

import pytest
import torch

from test_gpu_parity import DEV, rand_bf16

pytestmark = pytest.mark.gpu

OURS = ("ln_modulate", "rga", "qk_", "gelu", "mod_", "temb")


@pytest.fixture(scope="module")
def ops():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import modulate_ln_amd as m

    m._native.lib()  # fail loudly if the library is missing
    return m


def device_kernels(call):
    """Names of the device kernels that run during call()."""
    from torch.autograd import DeviceType
    from torch.profiler import ProfilerActivity, profile

    torch.cuda.synchronize()
    with profile(activities=[ProfilerActivity.CUDA], acc_events=True) as prof:
        call()
        torch.cuda.synchronize()
    return [e.name for e in prof.events() if e.device_type == DeviceType.CUDA]


def calls(ops):
    g = torch.Generator().manual_seed(3)
    B, S, D = 2, 256, 1024
    x = rand_bf16((B, S, D), g).to(DEV)
    xt = rand_bf16((B, D, S), g).to(DEV).transpose(1, 2)  # transposed storage, token stride 1
    sc = rand_bf16((B, D), g, std=0.1).to(DEV)
    sh = rand_bf16((B, D), g, std=0.1).to(DEV)
    gate = rand_bf16((B, D), g, std=0.5).to(DEV)
    upd = rand_bf16((B, S, D), g).to(DEV)
    q = rand_bf16((B, S, 8, 128), g).to(DEV)
    k = rand_bf16((B, S, 8, 128), g).to(DEV)
    w = tuple(rand_bf16((128,), g, std=0.05).to(DEV) for _ in range(4))
    qs = torch.tensor([0.25], dtype=torch.float32, device=DEV)
    h = rand_bf16((512, 3072), g).to(DEV)
    bias = rand_bf16((3072,), g, std=0.1).to(DEV)
    table = torch.randn((6, D), generator=g).to(DEV)
    temb = rand_bf16((B, S, 6, D), g).to(DEV)
    ws = ops.ln_modulate_workspace(xt)
    long_x = rand_bf16((1, 16, 16384), g).to(DEV)
    long_s = rand_bf16((1, 16384), g, std=0.1).to(DEV)
    return {
        "ln_modulate": ops.ln_modulate(x, sc, sh, 1e-6, prepare=True),
        "ln_modulate transposed": ops.ln_modulate(xt, sc, sh, 1e-6, prepare=True),
        "ln_modulate_ws transposed": ops.ln_modulate(xt, sc, sh, 1e-6, workspace=ws, prepare=True),
        "ln_modulate_noalloc transposed": ops.ln_modulate_noalloc(xt, sc, sh, 1e-6, out=torch.empty_like(x),
                                                                  prepare=True),
        "ln_modulate long rows": ops.ln_modulate(long_x, long_s, long_s, 1e-6, prepare=True),
        "ln_modulate_fold": ops.ln_modulate_fold(x, sc, sh, 1e-6, prepare=True),
        "ln_modulate_fp8": ops.ln_modulate_fp8(x, sc, sh, qs, 1e-6, prepare=True),
        "rmsnorm_scale_shift": ops.rmsnorm_scale_shift(x, sc, sh, 1e-6, prepare=True),
        "residual_gate_add": ops.residual_gate_add(x, gate, upd, prepare=True),
        "residual_gate_add_ln_modulate": ops.residual_gate_add_ln_modulate(x, gate, upd, sc, sh, 1e-6,
                                                                           prepare=True),
        "qk_head_layernorm": ops.qk_head_layernorm(q, k, *w, 1e-6, prepare=True),
        "qk_rmsnorm": ops.qk_rmsnorm(q, k, w[0], w[2], 1e-6, prepare=True),
        "bias_gelu_tanh": ops.bias_gelu_tanh(h, bias, prepare=True),
        "modulate_scale_shift": ops.modulate_scale_shift(x, sc, sh, prepare=True),
        "temb_table_slices": ops.temb_table_slices(table, temb, prepare=True),
    }


def test_one_dispatch_per_call(ops):
    prepared = calls(ops)
    for p in prepared.values():  # first calls out of the way (module loads, lookups)
        p()
    torch.cuda.synchronize()
    for name, p in prepared.items():
        ks = device_kernels(p)
        assert len(ks) == 1, (name, ks)
        assert any(t in ks[0] for t in OURS), (name, ks)


def test_kernel_choice(ops):
    """The launch shape each layout class and size takes (on this device's compute units):
    16-wave tabled blocks when they fill the chip with one row per wave, 4-wave prefetching
    ones for more rows, the row kernels when they would not fill it, the
    shared-table long-row kernel when its blocks fill three quarters of it, the workspace
    kernel for transposed storage given a workspace."""
    g = torch.Generator().manual_seed(5)
    cus = torch.cuda.get_device_properties(0).multi_processor_count

    def ln(B, S, D):
        x = rand_bf16((B, S, D), g).to(DEV)
        s = rand_bf16((B, D), g, std=0.1).to(DEV)
        return ops.ln_modulate(x, s, s, 1e-6, prepare=True)

    def fused(B, S, D):
        x = rand_bf16((B, S, D), g).to(DEV)
        s = rand_bf16((B, D), g, std=0.1).to(DEV)
        return ops.residual_gate_add_ln_modulate(x, s, x.clone(), s, s, 1e-6, prepare=True)

    xt = rand_bf16((2, 2240, 1024), g).to(DEV).transpose(1, 2)
    s2 = rand_bf16((2, 2240), g, std=0.1).to(DEV)
    many = 16 * cus  # rows of 4096: 16-wave blocks, one per compute unit
    long_rows = 4 * ((3 * cus + 3) // 4)  # rows of 16384: 4 per block, three quarters of the chip
    half_rows = 2 * ((4 * cus + 4) // 5)  # 2 per 8-wave block fill 80 % of the chip, 4 per block too few
    past_round = 4 * (cus + cus // 8)  # 4 per block: one round and an eighth
    expect = [
        ("half-size shared tables", ln(1, half_rows, 16384), "ln_modulate_mwt<8, true, false, 0, 512>"),
        ("nearly empty last round", ln(1, past_round, 16384), "ln_modulate_mw<"),
        ("fused half-size shared tables", fused(1, half_rows, 16384), "rga_ln_modulate_mwt<8, true, 512>"),
        ("tabled", ln(1, many, 4096), "ln_modulate_tab<8, 8, true, false, 0, false>"),
        ("tabled, more rows than waves", ln(1, many + 64, 4096), "ln_modulate_tab<8, 8, true, false, 0, true>"),
        ("few rows", ln(1, 128, 4096), "ln_modulate_rows<"),
        ("shared tables", ln(1, long_rows, 16384), "ln_modulate_mwt<8, true, false, 0, 1024>"),
        ("few long rows", ln(1, 128, 16384), "ln_modulate_mw<"),
        ("workspace", ops.ln_modulate(xt, s2, s2, 1e-6, workspace=ops.ln_modulate_workspace(xt), prepare=True),
         "ln_modulate_trc<"),
        ("transposed tiles", ops.ln_modulate(xt, s2, s2, 1e-6, prepare=True), "ln_modulate_tr<"),
        ("fused tabled", fused(1, many, 4096), "rga_ln_modulate_tab<8, 8, true, false>"),
        ("fused tabled, more rows than waves", fused(1, many + 64, 4096), "rga_ln_modulate_tab<8, 8, true, true>"),
        ("fused few rows", fused(1, 128, 4096), "rga_ln_modulate_mw<"),
        ("fused shared tables", fused(1, long_rows, 16384), "rga_ln_modulate_mwt<8, true, 1024>"),
    ]
    for name, p, kernel in expect:
        p()
    torch.cuda.synchronize()
    for name, p, kernel in expect:
        ks = device_kernels(p)
        assert len(ks) == 1 and kernel in ks[0], (name, kernel, ks)
