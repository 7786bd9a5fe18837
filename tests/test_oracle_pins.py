"""Pins of the CPU oracle against things other than itself: library routines,
closed forms, exact rational arithmetic, invariants.  CPU only.

The pages print no worked numeric example for the chain, so the fixed values
used here are closed forms derived from the definitions (written out in
tests/golden/closed_forms.txt with their derivations).
"""

from __future__ import annotations

import math
from decimal import Decimal, getcontext
from fractions import Fraction

import numpy as np
import pytest
import torch

from modulate_ln_amd import workloads as W

FP32, FP64 = 1, 0


def bits_of(t: torch.Tensor) -> np.ndarray:
    return W.bits(t)


def f32(bits) -> np.ndarray:
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def bf(vals) -> np.ndarray:
    """bf16 bits of values that are exactly representable."""
    t = torch.tensor(vals, dtype=torch.float32)
    assert torch.equal(t.to(torch.bfloat16).to(torch.float32), t), "not exact in bf16"
    return bits_of(t.to(torch.bfloat16))


# ---------------------------------------------------------------------------
# bf16 rounding
# ---------------------------------------------------------------------------

def test_bf16_from_f32_exhaustive_vs_torch(orc):
    """Every one of the 2^32 fp32 bit patterns: oracle RNE == torch CPU .to(bfloat16)
    (NaNs compared as NaN-ness only)."""
    n = 1 << 26
    base = np.arange(n, dtype=np.uint32)
    for chunk in range(1 << 6):
        u = base + np.uint32(chunk * n)
        f = u.view(np.float32)
        mine = orc.bf16_from_f32(f)
        ref = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        nan = np.isnan(f)
        assert np.array_equal(mine[~nan], ref[~nan]), "chunk %d" % chunk
        assert np.all(np.isnan(f32(mine[nan])))


def _nearest_bf16_exact(x: Fraction) -> int:
    """bf16 bits (non-negative) nearest to x >= 0 by exact rational search, ties to even."""
    lo, hi = 0, 0x7F80
    val = lambda b: Fraction(float(np.uint32(b << 16).view(np.float32)))  # noqa: E731
    if x == 0:
        return 0
    while hi - lo > 1:
        mid = (lo + hi) // 2
        if val(mid) <= x:
            lo = mid
        else:
            hi = mid
    vlo = val(lo)
    vup = Fraction(2) ** 128 if lo + 1 == 0x7F80 else val(lo + 1)
    if x - vlo < vup - x:
        return lo
    if vup - x < x - vlo:
        return lo + 1
    return lo if lo % 2 == 0 else lo + 1


def test_bf16_from_f64_vs_exact_rationals(orc):
    rng = np.random.default_rng(1)
    samples = list(rng.standard_normal(400) * 10.0 ** rng.integers(-40, 38, 400))
    # values straddling bf16 midpoints by one double ulp, and exact midpoints
    for b in rng.integers(1, 0x7F7F, 200):
        lo = float(np.uint32(int(b) << 16).view(np.float32))
        hi = float(np.uint32((int(b) + 1) << 16).view(np.float32))
        mid = (lo + hi) / 2
        samples += [mid, math.nextafter(mid, 0), math.nextafter(mid, math.inf)]
    samples += [0.0, -0.0, 1e-45, 2.0 ** -134, 3.0 * 2.0 ** -135, 3.3895313892515355e38, 3.4e38, 1e300]
    for d in samples:
        got = int(orc._load().orc_bf16_from_f64(float(d)))
        want = _nearest_bf16_exact(Fraction(abs(d)))
        if math.copysign(1.0, d) < 0:
            want |= 0x8000
        assert got == want, (d, hex(got), hex(want))


def test_bf16_from_f64_matches_f32_path_on_floats(orc):
    rng = np.random.default_rng(2)
    f = rng.standard_normal(100000).astype(np.float32) * np.float32(3.0)
    assert np.array_equal(orc.bf16_from_f64(f.astype(np.float64)), orc.bf16_from_f32(f))


# ---------------------------------------------------------------------------
# closed forms
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("mode", [FP64, FP32])
def test_worked_d4(orc, mode):
    """x = [-3,-1,1,3]: mean 0, var 5, x_hat = x/sqrt(5+eps) -> bf16 +-1.34375, +-0.447265625.
    With scale = 1 the factor 1+scale = 2 is exact, doubling the result."""
    x = bf([[-3.0, -1.0, 1.0, 3.0]])
    zero = bf([[0.0] * 4])
    one = bf([[1.0] * 4])
    out, mean, rstd = orc.ln_modulate(x, zero, zero, 1, 1e-6, mode, V=4, L=64)
    assert f32(out).tolist() == [[-1.34375, -0.447265625, 0.447265625, 1.34375]]
    assert mean[0] == 0.0
    assert abs(rstd[0] - 1 / math.sqrt(5 + 1e-6)) < 1e-7
    out2, _, _ = orc.ln_modulate(x, one, zero, 1, 1e-6, mode, V=4, L=64)
    assert f32(out2).tolist() == [[-2.6875, -0.89453125, 0.89453125, 2.6875]]
    # scale = -1 makes the factor 0: out = shift exactly
    sh = bf([[0.5, -0.25, 2.0, -8.0]])
    out3, _, _ = orc.ln_modulate(x, bf([[-1.0] * 4]), sh, 1, 1e-6, mode, V=4, L=64)
    assert np.array_equal(out3, sh)


@pytest.mark.parametrize("mode", [FP64, FP32])
@pytest.mark.parametrize("D", [4, 8, 12, 512, 2240, 4096, 4100])
@pytest.mark.parametrize("c", [0.0, 1.0, -3.5, 1000.0])
def test_constant_rows(orc, mode, D, c):
    """Constant row: mean = c exactly, var = 0, x_hat = +0, out = +0 with scale = shift = 0."""
    x = bf([[c] * D] * 2)
    z = bf([[0.0] * D])
    V = 8 if D % 8 == 0 else 4
    out, mean, rstd = orc.ln_modulate(x, z, z, 2, 1e-6, mode, V=V, L=64)
    assert np.all(out == 0)  # +0 bit pattern
    assert np.all(mean == c)
    eps32 = float(np.float32(1e-6))
    if mode == FP32:
        want = np.float32(1.0) / np.sqrt(np.float32(eps32))
        assert np.all(rstd == float(want))
    else:
        assert np.allclose(rstd, 1 / math.sqrt(eps32), rtol=1e-15)


@pytest.mark.parametrize("mode", [FP64, FP32])
def test_moments_of_xhat(orc, mode):
    """For random rows with var >> eps: mean(x_hat) ~ 0, var(x_hat) ~ var/(var+eps) ~ 1."""
    g = torch.Generator().manual_seed(3)
    x = (torch.randn(64, 2240, generator=g) * 4 + 1.5).to(torch.bfloat16)
    z = torch.zeros(1, 2240, dtype=torch.bfloat16)
    out, _, _ = orc.ln_modulate(bits_of(x), bits_of(z), bits_of(z), 64, 1e-6, mode, V=8, L=64)
    xh = f32(out).astype(np.float64)
    assert np.all(np.abs(xh.mean(axis=1)) <= 2.0 ** -8)
    assert np.all(np.abs(xh.var(axis=1) - 1.0) <= 2.0 ** -7)


def test_shift_invariance_fp64_bitwise(orc):
    """Integer rows in [-64, 64], D a power of two: the mean is exact in double, so
    LN(x + 64) and LN(x) are bit-identical in the two-pass mode."""
    rng = np.random.default_rng(4)
    for D in (64, 512, 4096):
        xi = rng.integers(-64, 65, size=(8, D)).astype(np.float32)
        a = orc.bf16_from_f32(xi)
        b = orc.bf16_from_f32(xi + 64.0)
        z = bf([[0.0] * D])
        oa, ma, ra = orc.ln_modulate(a, z, z, 8, 1e-6, FP64)
        ob, mb, rb = orc.ln_modulate(b, z, z, 8, 1e-6, FP64)
        assert np.array_equal(oa, ob)
        assert np.array_equal(ra, rb)
        assert np.array_equal(mb - ma, np.full(8, 64.0))


def test_shift_invariance_fp32_close(orc):
    rng = np.random.default_rng(5)
    xi = rng.integers(-64, 65, size=(16, 2240)).astype(np.float32)
    a = orc.bf16_from_f32(xi)
    b = orc.bf16_from_f32(xi + 64.0)
    ma, ra = orc.layernorm_stats(a, 1e-6, FP32)
    mb, rb = orc.layernorm_stats(b, 1e-6, FP32)
    assert np.allclose(mb - ma, 64.0, rtol=0, atol=1e-4)
    assert np.allclose(ra, rb, rtol=1e-5)


# ---------------------------------------------------------------------------
# Welford and the merge against exact rational arithmetic
# ---------------------------------------------------------------------------

def _exact_stats(vals):
    fr = [Fraction(float(v)) for v in vals]
    n = len(fr)
    mu = sum(fr) / n
    m2 = sum((v - mu) ** 2 for v in fr)
    return mu, m2


def test_welford_seq_vs_fractions(orc):
    rng = np.random.default_rng(6)
    for n in (1, 2, 3, 5, 7, 16, 100, 1000):
        for _ in range(5):
            x = rng.integers(-50, 51, n).astype(np.float32) * np.float32(0.25) + np.float32(rng.integers(-4, 5))
            m, m2 = orc.welford_seq(x)
            mu, M2 = _exact_stats(x)
            scale = float(max(abs(x).max(), 1.0))
            assert abs(float(m) - float(mu)) <= 4 * n * 2 ** -24 * scale
            assert abs(float(m2) - float(M2)) <= 8 * n * 2 ** -24 * (float(M2) + n * scale * scale * 2 ** -10) + 1e-30


def test_welford_small_exact_cases(orc):
    m, m2 = orc.welford_seq(np.array([3.0], np.float32))
    assert (m, m2) == (3.0, 0.0)
    m, m2 = orc.welford_seq(np.array([1.0, 3.0], np.float32))
    assert (m, m2) == (2.0, 2.0)  # mean (a+b)/2, m2 = (b-a)^2/2


def test_combine_identities(orc):
    a = np.array([1.5, 4.0, 3.0], np.float32)
    empty = np.zeros(3, np.float32)
    assert orc.welford_combine(a, empty) == tuple(a)
    assert orc.welford_combine(empty, a) == tuple(a)
    # two singletons a, b: mean (a+b)/2, m2 (b-a)^2/2, exact for small integers
    for x, y in ((1.0, 3.0), (-5.0, 7.0), (2.0, 2.0), (100.0, -28.0)):
        got = orc.welford_combine(np.array([x, 0, 1], np.float32), np.array([y, 0, 1], np.float32))
        assert got == ((x + y) / 2, (y - x) ** 2 / 2, 2.0)


def test_combine_vs_fractions(orc):
    rng = np.random.default_rng(7)
    for _ in range(200):
        na, nb = int(rng.integers(1, 40)), int(rng.integers(1, 40))
        xa = (rng.standard_normal(na) * 3 + 1).astype(np.float32)
        xb = (rng.standard_normal(nb) * 3 + 1).astype(np.float32)
        ma, m2a = orc.welford_seq(xa)
        mb, m2b = orc.welford_seq(xb)
        m, m2, n = orc.welford_combine(np.array([ma, m2a, na], np.float32), np.array([mb, m2b, nb], np.float32))
        mu, M2 = _exact_stats(np.concatenate([xa, xb]))
        assert n == na + nb
        assert abs(float(m) - float(mu)) <= 1e-5 * 4
        assert abs(float(m2) - float(M2)) <= 1e-5 * float(M2) + 1e-5


@pytest.mark.parametrize("L", [1, 2, 16, 64])
def test_fp32_stats_vs_fractions(orc, L):
    """Row statistics in the fixed order agree with exact rationals within fp32 error."""
    rng = np.random.default_rng(8)
    for D in (4, 12, 16, 64, 520):
        x = (rng.standard_normal((3, D)) * 2 - 0.5).astype(np.float32)
        xb = orc.bf16_from_f32(x)
        V = 8 if D % 8 == 0 else 4
        mean, rstd = orc.layernorm_stats(xb, 1e-6, FP32, V=V, L=L)
        for r in range(3):
            mu, M2 = _exact_stats(f32(xb[r]))
            var = M2 / D
            ex_rstd = 1.0 / math.sqrt(float(var) + float(np.float32(1e-6)))
            assert abs(mean[r] - float(mu)) <= 1e-5 * (1 + abs(float(mu)))
            assert abs(rstd[r] - ex_rstd) <= 1e-5 * ex_rstd


def test_fp64_stats_vs_fractions(orc):
    rng = np.random.default_rng(9)
    for D in (4, 16, 64):
        x = orc.bf16_from_f32((rng.standard_normal((4, D)) * 3).astype(np.float32))
        mean, rstd = orc.layernorm_stats(x, 1e-6, FP64)
        for r in range(4):
            mu, M2 = _exact_stats(f32(x[r]))
            getcontext().prec = 50
            var = Decimal(M2.numerator) / Decimal(M2.denominator) / D + Decimal(float(np.float32(1e-6)))
            ex = float(1 / var.sqrt())
            assert abs(mean[r] - float(mu)) <= 2 ** -50 * (1 + abs(float(mu)))
            assert abs(rstd[r] - ex) <= 1e-14 * ex


# ---------------------------------------------------------------------------
# special cases that reduce to library routines
# ---------------------------------------------------------------------------

def _midpoint_margin(vals: np.ndarray) -> np.ndarray:
    """distance of each value from the nearest bf16 rounding midpoint, in units of |value|"""
    f = vals.astype(np.float32)
    u = f.view(np.uint32)
    lo = (u & np.uint32(0xFFFF0000)).view(np.float32).astype(np.float64)
    hi = ((u & np.uint32(0xFFFF0000)) + np.uint32(0x10000)).view(np.float32).astype(np.float64)
    mid = (lo + hi) / 2
    return np.abs(vals - mid) / np.maximum(np.abs(vals), 1e-300)


def test_fp64_mode_equals_torch_layer_norm(orc):
    """scale = shift = 0: the chain is bf16(LN(x)); torch's float64 layer_norm rounded to
    bf16 must agree except where the double value sits within 1e-12 of a bf16 midpoint."""
    g = torch.Generator().manual_seed(10)
    x = (torch.randn(128, 2240, generator=g) * 4).to(torch.bfloat16)
    z = torch.zeros(1, 2240, dtype=torch.bfloat16)
    out, _, _ = orc.ln_modulate(bits_of(x), bits_of(z), bits_of(z), 128, 1e-6, FP64)
    ref64 = torch.nn.functional.layer_norm(x.double(), (2240,), eps=float(np.float32(1e-6))).numpy()
    ref = orc.bf16_from_f64(ref64)
    diff = out != ref
    assert np.all(_midpoint_margin(ref64[diff]) < 1e-12)
    assert diff.mean() < 1e-4


def test_elementwise_tail_equals_torch_eager(orc):
    """Given the oracle's own fp32 mean/rstd, the rest of ln_modulate is torch's eager bf16
    chain: bf16((x - mean) * rstd), then (1 + scale), *, + shift as bf16 tensor ops."""
    wl = W.glm_square(seed=11, S=64, D=4096)
    x, sc, sh = wl.tensors["x"], wl.tensors["scale"], wl.tensors["shift"]
    xb = bits_of(x.reshape(64, 4096))
    out, mean, rstd = orc.ln_modulate(xb, bits_of(sc), bits_of(sh), 64, 1e-5, FP32)
    xf = x.reshape(64, 4096).float()
    m = torch.from_numpy(mean.astype(np.float32))[:, None]
    r = torch.from_numpy(rstd.astype(np.float32))[:, None]
    xhat = ((xf - m) * r).to(torch.bfloat16)
    eager = xhat * (1 + sc) + sh
    assert np.array_equal(out, bits_of(eager))


@pytest.mark.parametrize("mode", [FP64, FP32])
def test_residual_gate_add_equals_torch_eager(orc, mode):
    """The gated residual is two bf16 tensor ops: torch CPU eager is the reference."""
    g = torch.Generator().manual_seed(12)
    B, S, D = 3, 17, 520
    res = torch.randn(B, S, D, generator=g).to(torch.bfloat16)
    upd = (torch.randn(B, S, D, generator=g) * 5).to(torch.bfloat16)
    gate = (torch.randn(B, D, generator=g) * 0.1).to(torch.bfloat16)
    eager = res + gate[:, None, :] * upd
    out = orc.residual_gate_add(bits_of(res.reshape(B * S, D)), bits_of(gate), bits_of(upd.reshape(B * S, D)), S, mode)
    assert np.array_equal(out, bits_of(eager.reshape(B * S, D)))
    # gate = 0 and update >= 0: t = +0, so out = residual except -0 + +0 = +0
    res[0, 0, :4] = torch.tensor([-0.0, 0.0, 1.0, -2.0])
    upd = upd.abs()
    zero = torch.zeros(B, D, dtype=torch.bfloat16)
    out0 = orc.residual_gate_add(bits_of(res.reshape(B * S, D)), bits_of(zero), bits_of(upd.reshape(B * S, D)), S, mode)
    want = bits_of(res.reshape(B * S, D)).copy()
    want[want == 0x8000] = 0
    assert np.array_equal(out0, want)


@pytest.mark.parametrize("mode", [FP64, FP32])
def test_qk_identity_affine_equals_no_affine(orc, mode):
    g = torch.Generator().manual_seed(13)
    x = torch.randn(96, 128, generator=g).to(torch.bfloat16)
    one = torch.ones(128, dtype=torch.bfloat16)
    zero = torch.zeros(128, dtype=torch.bfloat16)
    a = orc.qk_head_layernorm(bits_of(x), bits_of(one), bits_of(zero), 1e-6, mode)
    b = orc.qk_head_layernorm(bits_of(x), None, None, 1e-6, mode)
    assert np.array_equal(a, b)


def test_qk_fp64_equals_torch_affine_layer_norm(orc):
    wl = W.glm_qk(seed=14, S=8, H=32)
    q = wl.tensors["q"].reshape(-1, 128)
    w, b = wl.tensors["wq"], wl.tensors["bq"]
    out = orc.qk_head_layernorm(bits_of(q), bits_of(w), bits_of(b), 1e-6, FP64)
    ref64 = torch.nn.functional.layer_norm(q.double(), (128,), w.double(), b.double(), eps=float(np.float32(1e-6))).numpy()
    ref = orc.bf16_from_f64(ref64)
    diff = out != ref
    assert np.all(_midpoint_margin(ref64[diff]) < 1e-12)


def test_qk_fp32_within_one_ulp_of_fp64(orc):
    """The fixed-order fp32 statistics move an affine head output by at most one bf16 ulp."""
    wl = W.glm_qk(seed=16, S=16, H=32)
    k = wl.tensors["k"].reshape(-1, 128)
    w, b = wl.tensors["wk"], wl.tensors["bk"]
    a = f32(orc.qk_head_layernorm(bits_of(k), bits_of(w), bits_of(b), 1e-6, FP32)).astype(np.float64)
    r = f32(orc.qk_head_layernorm(bits_of(k), bits_of(w), bits_of(b), 1e-6, FP64)).astype(np.float64)
    ulp = np.maximum(np.abs(r), 2.0 ** -126) * 2.0 ** -7
    assert np.all(np.abs(a - r) <= ulp)
    assert np.mean(a != r) < 0.01


def test_gelu_f64_vs_torch(orc):
    z = np.linspace(-6, 6, 4001)
    ref = torch.nn.functional.gelu(torch.from_numpy(z), approximate="tanh").numpy()
    got = np.array([orc.gelu_tanh_f64(v) for v in z])
    assert np.allclose(got, ref, rtol=1e-12, atol=1e-15)


def test_gelu_f64_tail_vs_decimal(orc):
    """Large negative z, where 1 + tanh(u) cancels in double: 50-digit decimal reference."""
    getcontext().prec = 60
    k0 = (Decimal(2) / Decimal("3.14159265358979323846264338327950288419716939937510")).sqrt()
    for zf in (-4.0, -6.5, -9.0, -10.25, -12.0):
        zd = Decimal(zf)
        u = k0 * (zd + Decimal("0.044715") * zd ** 3)
        t = (2 * u).exp()  # 0.5 (1 + tanh u) = e^{2u} / (1 + e^{2u})
        exact = zd * t / (1 + t)
        got = orc.gelu_tanh_f64(zf)
        assert abs(Decimal(got) - exact) <= abs(exact) * Decimal("1e-13")


def test_bias_gelu_rounds_after_bias(orc):
    """z = bf16(x + bias) then gelu: with bias = 0 the gelu input is x itself."""
    g = torch.Generator().manual_seed(15)
    x = torch.randn(4, 64, generator=g).to(torch.bfloat16)
    zero = torch.zeros(64, dtype=torch.bfloat16)
    out, val = orc.bias_gelu_tanh(bits_of(x), bits_of(zero))
    ref = torch.nn.functional.gelu(x.double(), approximate="tanh").numpy()
    assert np.allclose(val, ref, rtol=1e-12, atol=1e-300)
    # a bias that changes the rounding of x + bias: z must be the bf16 sum
    xb = torch.full((1, 2), 1.0, dtype=torch.bfloat16)
    bias = torch.tensor([2.0 ** -9, 3 * 2.0 ** -9], dtype=torch.bfloat16)  # 1 + 2^-9 ties to 1, 1 + 3*2^-9 -> 1 + 2^-7
    _, v = orc.bias_gelu_tanh(bits_of(xb), bits_of(bias))
    assert v[0, 0] == orc.gelu_tanh_f64(1.0)
    assert v[0, 1] == orc.gelu_tanh_f64(1.0 + 2.0 ** -7)


def _mode_pin_rows(name):
    """(rows [R, D] bf16 bits, eps, V, L) of each workload shape, in the orders the kernels use:
    V = 8 (4 when D % 8 != 0) elements per vector; L = 64 lanes per row of up to 4096 elements,
    64 W for longer rows held by W waves, 16 per q/k head."""
    if name == "c1 (1,256,512)":
        wl = W.ln_small()
        return bits_of(wl.tensors["x"].reshape(-1, 512)), 1e-6, 8, 64
    if name == "c2 (2,1024,2240) tail D":
        wl = W.sana_transposed()
        xt = wl.tensors["xt"]  # [B, D, S] storage; logical rows are x[b, s, :]
        return bits_of(xt.transpose(1, 2).reshape(-1, xt.shape[1])), 1e-6, 8, 64
    if name == "c3 (1,4096,4096) outliers":
        wl = W.glm_square()
        return bits_of(wl.tensors["x"].reshape(-1, 4096)), 1e-5, 8, 64
    if name == "c4 heads Dh=128, L=16":
        wl = W.glm_qk(S=160)
        return bits_of(torch.cat([wl.tensors["q"], wl.tensors["k"]]).reshape(-1, 128)), 1e-6, 8, 16
    if name == "c5 (4,4096,3072) chain input":
        wl = W.dit_chain(S=512, blocks=1)
        return bits_of(wl.tensors["x"].reshape(-1, 3072)), 1e-6, 8, 64
    g = torch.Generator().manual_seed(hash(name) % 1000)
    D, L = {"D=4100, V=4, W=2": (4100, 128), "D=16384, W=4": (16384, 256),
            "D=65532, V=4, W=16": (65532, 1024)}[name]
    x = W.normal((48, D), g, mean=0.5, std=3.0)
    return bits_of(x), 1e-6, (8 if D % 8 == 0 else 4), L


@pytest.mark.parametrize("name", ["c1 (1,256,512)", "c2 (2,1024,2240) tail D", "c3 (1,4096,4096) outliers",
                                  "c4 heads Dh=128, L=16", "c5 (4,4096,3072) chain input", "D=4100, V=4, W=2",
                                  "D=16384, W=4", "D=65532, V=4, W=16"])
def test_fp32_mode_close_to_fp64_mode(orc, name):
    """The two statistics modes agree within the stated tolerances on every workload shape and
    every reduction order the kernels use: |dmean| <= 1e-5 sqrt(mean^2 + sigma^2) and
    |drstd| <= 1e-5 rstd against the fp64 two-pass definition."""
    xb, eps, V, L = _mode_pin_rows(name)
    m32, r32 = orc.layernorm_stats(xb, eps, FP32, V=V, L=L)
    m64, r64 = orc.layernorm_stats(xb, eps, FP64)
    sig = 1 / r64
    assert np.all(np.abs(m32 - m64) <= 1e-5 * np.sqrt(m64 ** 2 + sig ** 2)), name
    assert np.all(np.abs(r32 - r64) <= 1e-5 * r64), name
    # and the order matters only within that tolerance: another lane count moves the bits of
    # some rows (the pin would catch an oracle that ignored V or L)
    m32b, _ = orc.layernorm_stats(xb, eps, FP32, V=4 if V == 8 else V, L=L * 2 if L < 1024 else L // 2)
    assert np.all(np.abs(m32b - m64) <= 1e-5 * np.sqrt(m64 ** 2 + sig ** 2)), name


# ---------------------------------------------------------------------------
# residual_gate_add_ln_modulate: the gated residual update feeding ln_modulate
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("mode", [FP64, FP32])
def test_fused_residual_worked_d4(orc, mode):
    """Three inputs whose updated residual is [-3,-1,1,3] (exact in bf16): the normalized
    output is the worked closed form of the plain ln_modulate (x / sqrt(5 + eps))."""
    want = [[-1.34375, -0.447265625, 0.447265625, 1.34375]]
    zero = bf([[0.0] * 4])
    cases = [
        (bf([[0.0] * 4]), bf([[2.0] * 4]), bf([[-1.5, -0.5, 0.5, 1.5]])),  # 0 + 2*u
        (bf([[1.0] * 4]), bf([[1.0] * 4]), bf([[-4.0, -2.0, 0.0, 2.0]])),  # 1 + u
        (bf([[-3.0, -1.0, 1.0, 3.0]]), zero, bf([[7.0, -7.0, 0.5, 9.0]])),  # gate 0: residual
    ]
    for res, gate, upd in cases:
        r_out, out, mean, rstd = orc.residual_gate_add_ln_modulate(res, gate, upd, zero, zero, 1, 1e-6, mode,
                                                                   V=4, L=64)
        assert f32(r_out).tolist() == [[-3.0, -1.0, 1.0, 3.0]]
        assert f32(out).tolist() == want
        assert mean[0] == 0.0
        assert abs(rstd[0] - 1 / math.sqrt(5 + 1e-6)) < 1e-7
    # scale = 1 doubles it; gate = 0 with a -0 residual gives +0 in the new residual
    res = bf([[-3.0, -1.0, 1.0, 3.0]])
    r_out, out, _, _ = orc.residual_gate_add_ln_modulate(res, zero, bf([[1.0] * 4]), bf([[1.0] * 4]), zero, 1,
                                                         1e-6, mode, V=4, L=64)
    assert f32(out).tolist() == [[-2.6875, -0.89453125, 0.89453125, 2.6875]]
    res = bf([[-0.0, 2.0, -2.0, 0.0]])
    r_out, _, _, _ = orc.residual_gate_add_ln_modulate(res, zero, bf([[1.0] * 4]), zero, zero, 1, 1e-6, mode,
                                                       V=4, L=64)
    assert r_out.tolist() == [[0x0000, 0x4000, 0xC000, 0x0000]]


@pytest.mark.parametrize("mode", [FP64, FP32])
@pytest.mark.parametrize("D", [8, 2240])
def test_fused_residual_constant_rows(orc, mode, D):
    """residual c and update u with gate g such that c + g*u is constant: x_hat = +0, so out = +0
    with scale = shift = 0, and the updated residual is that constant."""
    res = bf([[1.0] * D, [-2.0] * D])
    upd = bf([[3.0] * D, [0.5] * D])
    gate = bf([[0.5] * D])
    z = bf([[0.0] * D])
    V = 8 if D % 8 == 0 else 4
    r_out, out, mean, _ = orc.residual_gate_add_ln_modulate(res, gate, upd, z, z, 2, 1e-6, mode, V=V, L=64)
    assert np.all(f32(r_out)[0] == 2.5) and np.all(f32(r_out)[1] == -1.75)
    assert np.all(out == 0)
    assert mean.tolist() == [2.5, -1.75]


def test_fused_residual_equals_torch_eager_chain(orc):
    """torch CPU eager is the reference for both outputs: the residual is two bf16 tensor ops;
    with scale = shift = 0 the output is float64 layer_norm of that residual rounded once
    (two-pass mode, up to values within 1e-12 of a bf16 midpoint); with real scale/shift,
    the tail after the oracle's own fp32 statistics is the eager bf16 chain."""
    g = torch.Generator().manual_seed(21)
    B, S, D = 2, 24, 2240
    res = torch.randn(B, S, D, generator=g).to(torch.bfloat16)
    upd = (torch.randn(B, S, D, generator=g) * 3).to(torch.bfloat16)
    gate = (torch.randn(B, D, generator=g) * 0.5).to(torch.bfloat16)
    sc = (torch.randn(B, D, generator=g) * 0.1).to(torch.bfloat16)
    sh = (torch.randn(B, D, generator=g) * 0.1).to(torch.bfloat16)
    xn = res + gate[:, None, :] * upd
    R = B * S
    flat = lambda t: bits_of(t.reshape(R, D))  # noqa: E731
    z = torch.zeros(B, D, dtype=torch.bfloat16)
    r_out, out, _, _ = orc.residual_gate_add_ln_modulate(flat(res), bits_of(gate), flat(upd), bits_of(z),
                                                         bits_of(z), S, 1e-6, FP64)
    assert np.array_equal(r_out, flat(xn))
    ref64 = torch.nn.functional.layer_norm(xn.double(), (D,), eps=float(np.float32(1e-6))).reshape(R, D).numpy()
    ref = orc.bf16_from_f64(ref64)
    diff = out != ref
    assert np.all(_midpoint_margin(ref64[diff]) < 1e-12)
    assert diff.mean() < 1e-4
    r_out, out, mean, rstd = orc.residual_gate_add_ln_modulate(flat(res), bits_of(gate), flat(upd), bits_of(sc),
                                                               bits_of(sh), S, 1e-6, FP32)
    assert np.array_equal(r_out, flat(xn))
    xf = xn.reshape(R, D).float()
    m = torch.from_numpy(mean.astype(np.float32))[:, None]
    r = torch.from_numpy(rstd.astype(np.float32))[:, None]
    xhat = ((xf - m) * r).to(torch.bfloat16).reshape(B, S, D)
    eager = xhat * (1 + sc[:, None, :]) + sh[:, None, :]
    assert np.array_equal(out, flat(eager))


# ---------------------------------------------------------------------------
# RMSNorm + scale/shift and per-head q/k RMSNorm
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("mode", [FP64, FP32])
def test_rms_worked_d4(orc, mode):
    """x = [-3,-1,1,3] has mean 0, so RMSNorm equals LayerNorm there; x = [3,4,3,4]:
    rinv = 1/sqrt(12.5 + eps) -> bf16 0.84765625, 1.1328125 (tests/golden/closed_forms.txt)."""
    zero = bf([[0.0] * 4])
    out, rinv = orc.rmsnorm_scale_shift(bf([[-3.0, -1.0, 1.0, 3.0]]), zero, zero, 1, 1e-6, mode, V=4, L=64)
    assert f32(out).tolist() == [[-1.34375, -0.447265625, 0.447265625, 1.34375]]
    assert abs(rinv[0] - 1 / math.sqrt(5 + 1e-6)) < 1e-7
    out, rinv = orc.rmsnorm_scale_shift(bf([[3.0, 4.0, 3.0, 4.0]]), zero, zero, 1, 1e-6, mode, V=4, L=64)
    assert f32(out).tolist() == [[0.84765625, 1.1328125, 0.84765625, 1.1328125]]
    assert abs(rinv[0] - 1 / math.sqrt(12.5 + 1e-6)) < 1e-7
    # scale = 1 doubles it exactly; scale = -1 leaves the shift
    out, _ = orc.rmsnorm_scale_shift(bf([[3.0, 4.0, 3.0, 4.0]]), bf([[1.0] * 4]), zero, 1, 1e-6, mode, V=4, L=64)
    assert f32(out).tolist() == [[1.6953125, 2.265625, 1.6953125, 2.265625]]
    sh = bf([[0.5, -0.25, 2.0, -8.0]])
    out, _ = orc.rmsnorm_scale_shift(bf([[3.0, 4.0, 3.0, 4.0]]), bf([[-1.0] * 4]), sh, 1, 1e-6, mode, V=4, L=64)
    assert np.array_equal(out, sh)


@pytest.mark.parametrize("mode", [FP64, FP32])
@pytest.mark.parametrize("D", [8, 2240, 4096])
def test_rms_constant_rows(orc, mode, D):
    """x = c: x_hat = c/sqrt(c^2 + eps) rounds to +-1 for |c| >= 1; c = 0 gives +0."""
    x = bf([[1.0] * D, [-3.5] * D, [1000.0] * D, [0.0] * D])
    z = bf([[0.0] * D])
    V = 8 if D % 8 == 0 else 4
    out, rinv = orc.rmsnorm_scale_shift(x, z, z, 4, 1e-6, mode, V=V, L=64)
    assert f32(out)[:3].tolist() == [[1.0] * D, [-1.0] * D, [1.0] * D]
    assert np.all(out[3] == 0)


def test_rms_fp64_mode_equals_torch_rms_norm(orc):
    """scale = shift = 0: the chain is bf16(RMSNorm(x)); torch's float64 rms_norm rounded to bf16
    must agree except where the double value sits within 1e-12 of a bf16 midpoint."""
    g = torch.Generator().manual_seed(30)
    x = (torch.randn(128, 2240, generator=g) * 3 + 0.5).to(torch.bfloat16)
    z = torch.zeros(1, 2240, dtype=torch.bfloat16)
    out, _ = orc.rmsnorm_scale_shift(bits_of(x), bits_of(z), bits_of(z), 128, 1e-6, FP64)
    ref64 = torch.nn.functional.rms_norm(x.double(), (2240,), eps=float(np.float32(1e-6))).numpy()
    ref = orc.bf16_from_f64(ref64)
    diff = out != ref
    assert np.all(_midpoint_margin(ref64[diff]) < 1e-12)
    assert diff.mean() < 1e-4


@pytest.mark.parametrize("mode", [FP64, FP32])
def test_rms_power_of_two_scale_invariance(orc, mode):
    """eps = 0: RMSNorm(2^k x) == RMSNorm(x) bit for bit (every step scales exactly)."""
    g = torch.Generator().manual_seed(31)
    x = (torch.randn(16, 1024, generator=g)).to(torch.bfloat16)
    z = torch.zeros(1, 1024, dtype=torch.bfloat16)
    base, r0 = orc.rmsnorm_scale_shift(bits_of(x), bits_of(z), bits_of(z), 16, 0.0, mode)
    for k in (-3, 5):
        xs = x * (2.0 ** k)
        out, r = orc.rmsnorm_scale_shift(bits_of(xs), bits_of(z), bits_of(z), 16, 0.0, mode)
        assert np.array_equal(out, base)
        assert np.array_equal(r * (2.0 ** k), r0)


def test_rms_stats_vs_fractions(orc):
    """Small-integer rows: the sum of squares is exact in both modes, so rinv is the correctly
    rounded (fp64) or within two fp32 roundings (fp32) of 1/sqrt(ss/D + eps), eps = 0."""
    rng = np.random.default_rng(32)
    for D in (4, 8, 12, 64, 200):
        xi = rng.integers(-20, 21, size=(3, D)).astype(np.float32)
        xi[:, 0] = 7  # no all-zero row
        x = bf(xi.tolist())
        z = bf([[0.0] * D])
        V = 8 if D % 8 == 0 else 4
        _, r32 = orc.rmsnorm_scale_shift(x, z, z, 3, 0.0, FP32, V=V, L=64)
        _, r64 = orc.rmsnorm_scale_shift(x, z, z, 3, 0.0, FP64)
        for i in range(3):
            ss = Fraction(int(np.sum(xi[i].astype(np.int64) ** 2)))
            exact = 1.0 / math.sqrt(float(ss / D))
            assert abs(r64[i] - exact) <= 2 * np.finfo(np.float64).eps * exact
            assert abs(r32[i] - exact) <= 4 * np.finfo(np.float32).eps * exact


def test_rms_tail_equals_torch_eager(orc):
    """Given the oracle's own fp32 rinv, the rest is torch's eager bf16 chain:
    bf16(x * rinv), then (1 + scale), *, + shift as bf16 tensor ops."""
    wl = W.glm_square(seed=33, S=64, D=4096)
    x, sc, sh = wl.tensors["x"], wl.tensors["scale"], wl.tensors["shift"]
    out, rinv = orc.rmsnorm_scale_shift(bits_of(x.reshape(64, 4096)), bits_of(sc), bits_of(sh), 64, 1e-5, FP32)
    xf = x.reshape(64, 4096).float()
    r = torch.from_numpy(rinv.astype(np.float32))[:, None]
    xhat = (xf * r).to(torch.bfloat16)
    eager = xhat * (1 + sc) + sh
    assert np.array_equal(out, bits_of(eager))


@pytest.mark.parametrize("mode", [FP64, FP32])
def test_qk_rms_unit_weight_equals_no_weight(orc, mode):
    g = torch.Generator().manual_seed(34)
    x = torch.randn(96, 128, generator=g).to(torch.bfloat16)
    one = torch.ones(128, dtype=torch.bfloat16)
    a = orc.qk_rmsnorm(bits_of(x), bits_of(one), 1e-6, mode)
    b = orc.qk_rmsnorm(bits_of(x), None, 1e-6, mode)
    assert np.array_equal(a, b)


def test_qk_rms_fp64_equals_torch_rms_norm(orc):
    """torch's float64 rms_norm with a weight, rounded once, against the fp64 mode."""
    g = torch.Generator().manual_seed(35)
    x = (torch.randn(512, 128, generator=g) * 2).to(torch.bfloat16)
    w = (1 + 0.05 * torch.randn(128, generator=g)).to(torch.bfloat16)
    out = orc.qk_rmsnorm(bits_of(x), bits_of(w), 1e-6, FP64)
    ref64 = torch.nn.functional.rms_norm(x.double(), (128,), weight=w.double(), eps=float(np.float32(1e-6))).numpy()
    ref = orc.bf16_from_f64(ref64)
    diff = out != ref
    assert np.all(_midpoint_margin(ref64[diff]) < 1e-12)
    assert diff.mean() < 1e-3


def test_qk_rms_fp32_equals_torch_fp32_tail(orc):
    """The fp32 mode's weight step is torch's fp32 arithmetic: (x * rinv) * w, rounded once."""
    g = torch.Generator().manual_seed(36)
    x = (torch.randn(256, 128, generator=g) * 2).to(torch.bfloat16)
    w = (1 + 0.05 * torch.randn(128, generator=g)).to(torch.bfloat16)
    z = torch.zeros(1, 128, dtype=torch.bfloat16)
    _, rinv = orc.rmsnorm_scale_shift(bits_of(x), bits_of(z), bits_of(z), 256, 1e-6, FP32, V=8, L=16)
    r = torch.from_numpy(rinv.astype(np.float32))[:, None]
    want = ((x.float() * r) * w.float()).to(torch.bfloat16)
    out = orc.qk_rmsnorm(bits_of(x), bits_of(w), 1e-6, FP32, V=8, L=16)
    assert np.array_equal(out, bits_of(want))


@pytest.mark.parametrize("norm", ["layer", "rms"])
def test_elementwise_tail_fp64_mode_equals_torch_eager(orc, norm):
    """The two-pass mode's tail: with x_hat = bf16(n) for the double-precision normalized value n
    (bf16_from_f64 is pinned on its own), the rest is torch's eager bf16 ops: (1 + scale), *,
    + shift -- each product and sum of two bf16 values is exact in double before its one rounding."""
    wl = W.glm_square(seed=37, S=64, D=4096)
    x, sc, sh = wl.tensors["x"], wl.tensors["scale"], wl.tensors["shift"]
    xb = bits_of(x.reshape(64, 4096))
    xd = x.reshape(64, 4096).double()
    if norm == "layer":
        out, mean, rstd = orc.ln_modulate(xb, bits_of(sc), bits_of(sh), 64, 1e-5, FP64)
        n = (xd - torch.from_numpy(mean)[:, None]) * torch.from_numpy(rstd)[:, None]
    else:
        out, rinv = orc.rmsnorm_scale_shift(xb, bits_of(sc), bits_of(sh), 64, 1e-5, FP64)
        n = xd * torch.from_numpy(rinv)[:, None]
    xhat = W.from_bits(orc.bf16_from_f64(n.numpy()))
    eager = xhat * (1 + sc) + sh
    assert np.array_equal(out, bits_of(eager))


# ---------------------------------------------------------------------------
# modulate_scale_shift and temb_table_slices
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("mode", [FP64, FP32])
def test_modulate_worked(orc, mode):
    """x = [1,2,3,4]: scale 1 doubles exactly and shift 0.5 is exact: [2.5, 4.5, 6.5, 8.5];
    scale -1 leaves the shift; scale 0, shift 0 returns x (every step exact)."""
    x = bf([[1.0, 2.0, 3.0, 4.0]])
    out = orc.modulate_scale_shift(x, bf([[1.0] * 4]), bf([[0.5] * 4]), 1, mode)
    assert f32(out).tolist() == [[2.5, 4.5, 6.5, 8.5]]
    sh = bf([[0.5, -0.25, 2.0, -8.0]])
    assert np.array_equal(orc.modulate_scale_shift(x, bf([[-1.0] * 4]), sh, 1, mode), sh)
    assert np.array_equal(orc.modulate_scale_shift(x, bf([[0.0] * 4]), bf([[0.0] * 4]), 1, mode), x)


@pytest.mark.parametrize("mode", [FP64, FP32])
@pytest.mark.parametrize("per_token", [False, True])
def test_modulate_equals_torch_eager(orc, mode, per_token):
    """x * (1 + scale) + shift as bf16 tensor ops on the CPU, adaLN rows per sample or per token."""
    g = torch.Generator().manual_seed(40)
    B, S, D = 3, 17, 520
    x = (torch.randn(B, S, D, generator=g) * 3).to(torch.bfloat16)
    shape = (B, S, D) if per_token else (B, 1, D)
    sc = (torch.randn(*shape, generator=g) * 0.5).to(torch.bfloat16)
    sh = (torch.randn(*shape, generator=g) * 0.5).to(torch.bfloat16)
    eager = x * (1 + sc) + sh
    rows = (lambda t: bits_of(t.reshape(B * S, D))) if per_token else (lambda t: bits_of(t[:, 0]))  # noqa: E731
    out = orc.modulate_scale_shift(bits_of(x.reshape(B * S, D)), rows(sc), rows(sh), S, mode)
    assert np.array_equal(out, bits_of(eager.reshape(B * S, D)))


@pytest.mark.parametrize("temb_f32", [False, True])
def test_temb_slices_equal_torch_chunks(orc, temb_f32):
    """(table + temb.float()).chunk(6, dim=2), each slice .contiguous(), on the CPU."""
    g = torch.Generator().manual_seed(41)
    B, L, M, D = 2, 9, 6, 520
    table = torch.randn(1, 1, M, D, generator=g) * 0.1
    temb = torch.randn(B, L, M, D, generator=g)
    if not temb_f32:
        temb = temb.to(torch.bfloat16)
    chunks = (table + temb.float()).chunk(M, dim=2)
    want = np.stack([c.contiguous().reshape(B, L, D).numpy() for c in chunks])
    t_in = temb.numpy() if temb_f32 else bits_of(temb)
    out = orc.temb_table_slices(table.reshape(M, D).numpy(), t_in, temb_is_f32=temb_f32)
    assert out.shape == (M, B, L, D)
    assert np.array_equal(out.view(np.uint32), want.view(np.uint32))


def test_temb_slices_zero_table_is_the_widening(orc):
    """A zero table returns float(temb) exactly, slice m holding temb[:, :, m]."""
    g = torch.Generator().manual_seed(42)
    temb = torch.randn(1, 5, 9, 64, generator=g).to(torch.bfloat16)
    out = orc.temb_table_slices(np.zeros((9, 64), np.float32), bits_of(temb))
    for m in range(9):
        assert np.array_equal(out[m, 0], temb[0, :, m].float().numpy())


# ---------------------------------------------------------------------------
# OCP FP8 E4M3 conversion, the FP8 producer and the single-rounding fold
# ---------------------------------------------------------------------------

def test_fp8_decode_table_vs_torch(orc):
    codes = np.arange(256, dtype=np.uint8)
    mine = orc.f64_from_fp8(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(mine), nan) and nan.sum() == 2
    assert np.array_equal(mine[~nan], ref[~nan])
    assert mine[0x7E] == 448.0 and mine[1] == 2.0 ** -9 and mine[0x08] == 2.0 ** -6


def test_fp8_encode_vs_torch(orc):
    """Every bf16 value as fp32, the exact midpoints between adjacent codes and one fp32 ulp
    either side, and 2M log-uniform fp32 values: nearest-even codes equal torch's conversion."""
    allbf = (np.arange(1 << 16, dtype=np.uint32) << np.uint32(16)).view(np.float32)
    vals = [allbf]
    codes = np.arange(0x7E, dtype=np.uint8)
    v = orc.f64_from_fp8(codes)
    mids = ((v[:-1] + v[1:]) / 2).astype(np.float32)
    mids = np.concatenate([mids, [np.float32(464.0)]])
    vals += [mids, np.nextafter(mids, np.float32(0)), np.nextafter(mids, np.float32(1e9)), v.astype(np.float32)]
    rng = np.random.default_rng(43)
    mag = (2.0 ** rng.uniform(-14, 9.2, 2_000_000)).astype(np.float32)
    vals.append(mag * np.where(rng.random(mag.size) < 0.5, -1, 1).astype(np.float32))
    a = np.concatenate(vals).astype(np.float32)
    a = np.concatenate([a, -a])
    mine = orc.fp8_from_f32(a)
    ref = torch.from_numpy(a).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    nan = np.isnan(a)
    assert np.array_equal(mine[~nan], ref[~nan])
    assert np.all((mine[nan] & 0x7F) == 0x7F)


@pytest.mark.parametrize("mode", [FP64, FP32])
def test_ln_modulate_fp8_worked(orc, mode):
    """tests/golden/closed_forms.txt: the worked row quantized with qscale 1 and 0.5."""
    x = bf([[-3.0, -1.0, 1.0, 3.0]])
    z = bf([[0.0] * 4])
    q, mean, rstd = orc.ln_modulate_fp8(x, z, z, 1, 1e-6, 1.0, mode, V=4, L=64)
    assert q.tolist() == [[0xBB, 0xAE, 0x2E, 0x3B]]
    assert mean[0] == 0.0
    q, _, _ = orc.ln_modulate_fp8(x, z, z, 1, 1e-6, 0.5, mode, V=4, L=64)
    assert q.tolist() == [[0xC3, 0xB6, 0x36, 0x43]]


@pytest.mark.parametrize("qscale", [0.0123, 0.25, 3.0])
def test_ln_modulate_fp8_tail_vs_torch(orc, qscale):
    """fp32 mode: the quantizer is torch's fp32 ops on the oracle's own bf16 output:
    (y * float32(1/s)).clamp(-448, 448).to(float8_e4m3fn).  With s a power of two the
    fp64 mode (exact quotient) gives the same codes."""
    wl = W.glm_square(seed=44, S=32, D=4096)
    x, sc, sh = wl.tensors["x"], wl.tensors["scale"], wl.tensors["shift"]
    xb = bits_of(x.reshape(32, 4096))
    y, _, _ = orc.ln_modulate(xb, bits_of(sc), bits_of(sh), 32, 1e-5, FP32)
    q, _, _ = orc.ln_modulate_fp8(xb, bits_of(sc), bits_of(sh), 32, 1e-5, qscale, FP32)
    inv = torch.tensor(1.0, dtype=torch.float32) / torch.tensor(qscale, dtype=torch.float32)
    yt = W.from_bits(y).float()
    want = (yt * inv).clamp(-448, 448).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(q, want)
    if qscale == 0.25:
        q64, _, _ = orc.ln_modulate_fp8(xb, bits_of(sc), bits_of(sh), 32, 1e-5, qscale, FP64)
        y64, _, _ = orc.ln_modulate(xb, bits_of(sc), bits_of(sh), 32, 1e-5, FP64)
        want64 = (W.from_bits(y64).float() * 4).clamp(-448, 448).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        assert np.array_equal(q64, want64)


@pytest.mark.parametrize("mode", [FP64, FP32])
def test_fold_worked(orc, mode):
    x = bf([[-3.0, -1.0, 1.0, 3.0]])
    z = bf([[0.0] * 4])
    out, _, _ = orc.ln_modulate_fold(x, z, z, 1, 1e-6, mode, V=4, L=64)
    assert f32(out).tolist() == [[-1.34375, -0.447265625, 0.447265625, 1.34375]]
    sh = bf([[0.5, -0.25, 2.0, -8.0]])
    out, _, _ = orc.ln_modulate_fold(x, bf([[-1.0] * 4]), sh, 1, 1e-6, mode, V=4, L=64)
    assert np.array_equal(out, sh)


def test_fold_fp64_mode_equals_torch_affine_layer_norm(orc):
    """layer_norm(x, weight=bf16(1 + scale), bias=shift) in float64, rounded once."""
    g = torch.Generator().manual_seed(45)
    x = (torch.randn(64, 2240, generator=g) * 2).to(torch.bfloat16)
    sc = (torch.randn(1, 2240, generator=g) * 0.3).to(torch.bfloat16)
    sh = (torch.randn(1, 2240, generator=g) * 0.3).to(torch.bfloat16)
    out, _, _ = orc.ln_modulate_fold(bits_of(x), bits_of(sc), bits_of(sh), 64, 1e-6, FP64)
    w = (1 + sc).to(torch.bfloat16).double()[0]
    ref64 = torch.nn.functional.layer_norm(x.double(), (2240,), weight=w, bias=sh.double()[0],
                                           eps=float(np.float32(1e-6))).numpy()
    ref = orc.bf16_from_f64(ref64)
    diff = out != ref
    assert np.all(_midpoint_margin(ref64[diff]) < 1e-12)
    assert diff.mean() < 1e-4


def _nearest_f32_exact(x: Fraction) -> float:
    """fp32 nearest to x (any sign) by exact rational search over bit patterns, ties to even."""
    if x < 0:
        return -_nearest_f32_exact(-x)
    lo, hi = 0, 0x7F800000
    val = lambda b: Fraction(float(np.uint32(b).view(np.float32)))  # noqa: E731
    while hi - lo > 1:
        mid = (lo + hi) // 2
        if val(mid) <= x:
            lo = mid
        else:
            hi = mid
    vlo, vup = val(lo), val(lo + 1)
    b = lo if (x - vlo < vup - x or (x - vlo == vup - x and lo % 2 == 0)) else lo + 1
    return float(np.uint32(b).view(np.float32))


def test_fold_fp32_tail_exact(orc):
    """fp32 mode: out = bf16(fma(w, n, b)) with a single rounding of w*n + b to fp32, checked
    against exact rational arithmetic from the oracle's own fp32 mean/rstd."""
    g = torch.Generator().manual_seed(46)
    R, D = 4, 512
    x = (torch.randn(R, D, generator=g) * 2).to(torch.bfloat16)
    sc = (torch.randn(1, D, generator=g) * 0.3).to(torch.bfloat16)
    sh = (torch.randn(1, D, generator=g) * 0.3).to(torch.bfloat16)
    out, mean, rstd = orc.ln_modulate_fold(bits_of(x), bits_of(sc), bits_of(sh), R, 1e-6, FP32)
    xf = x.float().numpy()
    n = (xf - mean.astype(np.float32)[:, None]) * rstd.astype(np.float32)[:, None]  # fp32 ops, RN each
    w = (1 + sc.float()).to(torch.bfloat16).float().numpy()[0]
    b = sh.float().numpy()[0]
    want = np.empty((R, D), dtype=np.float32)
    for i in range(R):
        for j in range(D):
            want[i, j] = _nearest_f32_exact(Fraction(float(w[j])) * Fraction(float(n[i, j])) + Fraction(float(b[j])))
    assert np.array_equal(out, orc.bf16_from_f32(want))
