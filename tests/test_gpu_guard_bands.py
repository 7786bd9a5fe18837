"""Guard bands: every output of every entry point is written into the middle
of a larger buffer whose surrounding bytes hold a known pattern; after the
call the pattern must be intact (no tail or overrun write past the output)
and the output must equal, byte for byte, that of the same call into a
freshly allocated tensor (which the parity tests check against the oracle).

Ragged shapes (D with a partial last vector step, odd row counts, D % 8 != 0)
and outputs placed off their natural vector alignment (a 2-byte offset for
bf16, 4 for fp32, 8 for FP8 bytes) drive the tail and narrow-vector paths.
"""

from __future__ import annotations

import pytest
import torch

from test_gpu_parity import DEV, rand_bf16

pytestmark = pytest.mark.gpu

PAD = 4096       # guard bytes on each side
PATTERN = 0xA5   # bf16 0xA5A5 and fp32 0xA5A5A5A5 are finite, FP8 0xA5 too


@pytest.fixture(scope="module")
def ops():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import modulate_ln_amd as m

    m._native.lib()
    return m


class Banded:
    """A tensor of the given shape and dtype at byte offset PAD + skew inside
    a pattern-filled byte buffer."""

    def __init__(self, shape, dtype, skew=0):
        n = 1
        for s in shape:
            n *= s
        item = torch.empty((), dtype=dtype).element_size()
        self.lo = PAD + skew
        self.nbytes = n * item
        self.raw = torch.full((self.lo + self.nbytes + PAD,), PATTERN, dtype=torch.uint8, device=DEV)
        self.t = self.raw[self.lo:self.lo + self.nbytes].view(dtype).view(shape)

    def check(self, what):
        torch.cuda.synchronize()
        raw = self.raw.cpu()
        before = raw[:self.lo]
        after = raw[self.lo + self.nbytes:]
        bad_b = int((before != PATTERN).sum())
        bad_a = int((after != PATTERN).sum())
        assert bad_b == 0 and bad_a == 0, "%s: %d guard bytes changed before, %d after" % (what, bad_b, bad_a)


def same_bytes(got, want, what, fp8=False):
    g = got.contiguous().view(torch.uint8).cpu()
    w = want.contiguous().view(torch.uint8).cpu()
    if fp8:  # NaN codes compare as NaN
        nan = ((g & 0x7F) == 0x7F) & ((w & 0x7F) == 0x7F)
        ok = (g == w) | nan
    else:
        ok = g == w
    assert bool(ok.all()), "%s: %d bytes differ from the unbanded call" % (what, int((~ok).sum()))


SHAPES = [(3, 37, 2240), (1, 5, 4100), (2, 3, 12), (1, 7, 4096), (2, 1, 520), (2, 3, 12296), (1, 2, 65532)]
SKEWS = {torch.bfloat16: (0, 2), torch.float32: (0, 4), torch.float8_e4m3fn: (0, 8)}


def ln_inputs(shape, seed, transposed=False):
    g = torch.Generator().manual_seed(seed)
    B, S, D = shape
    if transposed:
        x = rand_bf16((B, D, S), g).to(DEV).transpose(1, 2)
    else:
        x = rand_bf16((B, S, D), g).to(DEV)
    sc = rand_bf16((B, D), g, 0.1).to(DEV)
    sh = rand_bf16((B, D), g, 0.1).to(DEV)
    return x, sc, sh


def stats_pair(B, S, skew):
    return Banded((B * S,), torch.float32, skew), Banded((B * S,), torch.float32, skew)


@pytest.mark.parametrize("shape", SHAPES + [(2, 70, 2240)])
@pytest.mark.parametrize("op", ["ln_modulate", "ln_modulate_fold"])
@pytest.mark.parametrize("skew", [0, 1])
def test_ln_family_bands(ops, op, shape, skew):
    B, S, D = shape
    x, sc, sh = ln_inputs(shape, 11 + D, transposed=(S == 70))
    fn = getattr(ops, op)
    ref_m = torch.empty(B * S, dtype=torch.float32, device=DEV)
    ref_r = torch.empty(B * S, dtype=torch.float32, device=DEV)
    ref = fn(x, sc, sh, 1e-6, mean_out=ref_m, rstd_out=ref_r)
    o = Banded((B, S, D), torch.bfloat16, SKEWS[torch.bfloat16][skew])
    m, r = stats_pair(B, S, SKEWS[torch.float32][skew])
    fn(x, sc, sh, 1e-6, out=o.t, mean_out=m.t, rstd_out=r.t)
    what = "%s %s skew=%d" % (op, shape, skew)
    for band, want, name in ((o, ref, "out"), (m, ref_m, "mean"), (r, ref_r, "rstd")):
        band.check("%s %s" % (what, name))
        same_bytes(band.t, want, "%s %s" % (what, name))


@pytest.mark.parametrize("shape", SHAPES + [(2, 70, 2240)])
@pytest.mark.parametrize("skew", [0, 1])
def test_fp8_bands(ops, shape, skew):
    B, S, D = shape
    x, sc, sh = ln_inputs(shape, 23 + D, transposed=(S == 70))
    q = torch.tensor([0.05], dtype=torch.float32, device=DEV)
    ref_m = torch.empty(B * S, dtype=torch.float32, device=DEV)
    ref_r = torch.empty(B * S, dtype=torch.float32, device=DEV)
    ref = ops.ln_modulate_fp8(x, sc, sh, q, 1e-6, mean_out=ref_m, rstd_out=ref_r)
    # the FP8 output must be V-byte aligned (V = 8 when D % 8 == 0, else 4)
    sk = SKEWS[torch.float8_e4m3fn][skew] if D % 8 == 0 else 4 * skew
    o = Banded((B, S, D), torch.float8_e4m3fn, sk)
    m, r = stats_pair(B, S, SKEWS[torch.float32][skew])
    ops.ln_modulate_fp8(x, sc, sh, q, 1e-6, out=o.t, mean_out=m.t, rstd_out=r.t)
    what = "fp8 %s skew=%d" % (shape, skew)
    o.check(what + " out")
    same_bytes(o.t, ref, what + " out", fp8=True)
    for band, want, name in ((m, ref_m, "mean"), (r, ref_r, "rstd")):
        band.check("%s %s" % (what, name))
        same_bytes(band.t, want, "%s %s" % (what, name))


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("skew", [0, 1])
def test_rmsnorm_bands(ops, shape, skew):
    B, S, D = shape
    x, sc, sh = ln_inputs(shape, 31 + D)
    ref_r = torch.empty(B * S, dtype=torch.float32, device=DEV)
    ref = ops.rmsnorm_scale_shift(x, sc, sh, 1e-6, rinv_out=ref_r)
    o = Banded((B, S, D), torch.bfloat16, SKEWS[torch.bfloat16][skew])
    r = Banded((B * S,), torch.float32, SKEWS[torch.float32][skew])
    ops.rmsnorm_scale_shift(x, sc, sh, 1e-6, out=o.t, rinv_out=r.t)
    what = "rmsnorm %s skew=%d" % (shape, skew)
    for band, want, name in ((o, ref, "out"), (r, ref_r, "rinv")):
        band.check("%s %s" % (what, name))
        same_bytes(band.t, want, "%s %s" % (what, name))


@pytest.mark.parametrize("shape", SHAPES + [(1, 3, 7)])
@pytest.mark.parametrize("skew", [0, 1])
def test_residual_gate_add_bands(ops, shape, skew):
    B, S, D = shape
    g = torch.Generator().manual_seed(41 + D)
    res = rand_bf16((B, S, D), g).to(DEV)
    gate = rand_bf16((B, D), g, 0.1).to(DEV)
    upd = rand_bf16((B, S, D), g).to(DEV)
    ref = ops.residual_gate_add(res, gate, upd)
    o = Banded((B, S, D), torch.bfloat16, SKEWS[torch.bfloat16][skew])
    ops.residual_gate_add(res, gate, upd, out=o.t)
    what = "residual_gate_add %s skew=%d" % (shape, skew)
    o.check(what)
    same_bytes(o.t, ref, what)


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("skew", [0, 1])
def test_fused_residual_ln_bands(ops, shape, skew):
    B, S, D = shape
    g = torch.Generator().manual_seed(53 + D)
    res = rand_bf16((B, S, D), g).to(DEV)
    gate = rand_bf16((B, D), g, 0.1).to(DEV)
    upd = rand_bf16((B, S, D), g).to(DEV)
    sc = rand_bf16((B, D), g, 0.1).to(DEV)
    sh = rand_bf16((B, D), g, 0.1).to(DEV)
    ref_m = torch.empty(B * S, dtype=torch.float32, device=DEV)
    ref_r = torch.empty(B * S, dtype=torch.float32, device=DEV)
    ref_res, ref = ops.residual_gate_add_ln_modulate(res, gate, upd, sc, sh, 1e-6, mean_out=ref_m,
                                                     rstd_out=ref_r)
    sk = SKEWS[torch.bfloat16][skew]
    ro = Banded((B, S, D), torch.bfloat16, sk)
    o = Banded((B, S, D), torch.bfloat16, sk)
    m, r = stats_pair(B, S, SKEWS[torch.float32][skew])
    ops.residual_gate_add_ln_modulate(res, gate, upd, sc, sh, 1e-6, residual_out=ro.t, out=o.t,
                                      mean_out=m.t, rstd_out=r.t)
    what = "residual_gate_add_ln_modulate %s skew=%d" % (shape, skew)
    for band, want, name in ((ro, ref_res, "residual_out"), (o, ref, "out"), (m, ref_m, "mean"),
                             (r, ref_r, "rstd")):
        band.check("%s %s" % (what, name))
        same_bytes(band.t, want, "%s %s" % (what, name))


@pytest.mark.parametrize("shape", SHAPES + [(1, 3, 7)])
@pytest.mark.parametrize("per_token", [False, True])
@pytest.mark.parametrize("skew", [0, 1])
def test_modulate_bands(ops, shape, per_token, skew):
    B, S, D = shape
    g = torch.Generator().manual_seed(61 + D)
    x = rand_bf16((B, S, D), g).to(DEV)
    rows = (B, S, D) if per_token else (B, D)
    sc = rand_bf16(rows, g, 0.1).to(DEV)
    sh = rand_bf16(rows, g, 0.1).to(DEV)
    ref = ops.modulate_scale_shift(x, sc, sh)
    o = Banded((B, S, D), torch.bfloat16, SKEWS[torch.bfloat16][skew])
    ops.modulate_scale_shift(x, sc, sh, out=o.t)
    what = "modulate_scale_shift %s per_token=%s skew=%d" % (shape, per_token, skew)
    o.check(what)
    same_bytes(o.t, ref, what)


@pytest.mark.parametrize("B,L,M,D", [(1, 5, 6, 3072), (2, 3, 6, 2244), (1, 4, 2, 7)])
@pytest.mark.parametrize("temb_dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("skew", [0, 1])
def test_temb_bands(ops, B, L, M, D, temb_dtype, skew):
    g = torch.Generator().manual_seed(71 + D)
    table = torch.randn((M, D), generator=g).to(DEV)
    temb = torch.randn((B, L, M, D), generator=g).to(temb_dtype).to(DEV)
    ref = ops.temb_table_slices(table, temb)
    o = Banded((M, B, L, D), torch.float32, SKEWS[torch.float32][skew])
    ops.temb_table_slices(table, temb, out=o.t)
    what = "temb_table_slices %s %s skew=%d" % ((B, L, M, D), temb_dtype, skew)
    o.check(what)
    same_bytes(o.t, ref, what)


@pytest.mark.parametrize("Dh", [4, 12, 96, 128, 132, 256])
@pytest.mark.parametrize("op", ["qk_head_layernorm", "qk_rmsnorm"])
@pytest.mark.parametrize("skew", [0, 1])
def test_qk_bands(ops, op, Dh, skew):
    g = torch.Generator().manual_seed(83 + Dh)
    B, S, H = 2, 5, 3
    q = rand_bf16((B, S, H, Dh), g).to(DEV)
    k = rand_bf16((B, S, H, Dh), g).to(DEV)
    wq = rand_bf16((Dh,), g, 0.05).to(DEV) + 1
    wk = rand_bf16((Dh,), g, 0.05).to(DEV) + 1
    if op == "qk_head_layernorm":
        bq = rand_bf16((Dh,), g, 0.02).to(DEV)
        bk = rand_bf16((Dh,), g, 0.02).to(DEV)
        call = lambda **kw: ops.qk_head_layernorm(q, k, wq, bq, wk, bk, 1e-6, **kw)
    else:
        call = lambda **kw: ops.qk_rmsnorm(q, k, wq, wk, 1e-6, **kw)
    ref_q, ref_k = call()
    sk = SKEWS[torch.bfloat16][skew]
    qo = Banded((B, S, H, Dh), torch.bfloat16, sk)
    ko = Banded((B, S, H, Dh), torch.bfloat16, sk)
    call(q_out=qo.t, k_out=ko.t)
    what = "%s Dh=%d skew=%d" % (op, Dh, skew)
    for band, want, name in ((qo, ref_q, "q"), (ko, ref_k, "k")):
        band.check("%s %s" % (what, name))
        same_bytes(band.t, want, "%s %s" % (what, name))


@pytest.mark.parametrize("rows,width", [(3, 12288), (5, 4100), (7, 12), (2, 7)])
@pytest.mark.parametrize("skew", [0, 1])
def test_gelu_bands(ops, rows, width, skew):
    g = torch.Generator().manual_seed(97 + width)
    x = rand_bf16((rows, width), g).to(DEV)
    bias = rand_bf16((width,), g, 0.1).to(DEV)
    ref = ops.bias_gelu_tanh(x, bias)
    o = Banded((rows, width), torch.bfloat16, SKEWS[torch.bfloat16][skew])
    ops.bias_gelu_tanh(x, bias, out=o.t)
    what = "bias_gelu_tanh (%d,%d) skew=%d" % (rows, width, skew)
    o.check(what)
    same_bytes(o.t, ref, what)


@pytest.mark.parametrize("shape", [(2, 1024, 2240), (3, 1024, 2240), (1, 64, 8), (2, 128, 4096), (1, 192, 520)])
@pytest.mark.parametrize("skew", [0, 1])
def test_ln_modulate_workspace_bands(ops, shape, skew):
    """ln_modulate_ws on transposed storage: the output, the statistics and the workspace
    itself (zero-filled inside its bands) are written within their bounds only; skew 1
    puts the output off the 16-byte alignment the workspace path needs (ln_modulate's
    kernels then run, the workspace untouched)."""
    B, S, D = shape
    x, sc, sh = ln_inputs(shape, 41 + D, transposed=True)
    ref_m = torch.empty(B * S, dtype=torch.float32, device=DEV)
    ref_r = torch.empty(B * S, dtype=torch.float32, device=DEV)
    ref = ops.ln_modulate(x, sc, sh, 1e-6, mean_out=ref_m, rstd_out=ref_r)
    nb = ops.ln_modulate_workspace_size(x)
    assert nb > 0
    w = Banded((nb,), torch.uint8)
    w.t.zero_()
    o = Banded((B, S, D), torch.bfloat16, SKEWS[torch.bfloat16][skew])
    m, r = stats_pair(B, S, SKEWS[torch.float32][skew])
    for call in range(2):  # the second call finds the workspace as the first left it
        ops.ln_modulate(x, sc, sh, 1e-6, out=o.t, mean_out=m.t, rstd_out=r.t, workspace=w.t)
        what = "ln_modulate_ws %s skew=%d call %d" % (shape, skew, call)
        for band, want, name in ((o, ref, "out"), (m, ref_m, "mean"), (r, ref_r, "rstd")):
            band.check("%s %s" % (what, name))
            same_bytes(band.t, want, "%s %s" % (what, name))
        w.check("%s workspace" % what)
        if skew:
            assert not bool(w.t.any()), "%s: workspace written off the workspace path" % what
