"""Host-side checks of the C ABI: the library loads, exports every symbol the
header declares, and rejects bad arguments with the documented codes BEFORE
any HIP call (so these run without a GPU).  No compute call is made here:
every entry-point call below is one the validator rejects.
"""

from __future__ import annotations

import os
import re
import subprocess

import pytest

from modulate_ln_amd import _native as N

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "adaln.h")

# fake, never dereferenced device addresses (256-byte aligned, far apart)
P0, P1, P2, P3, P4 = (0x10000000 * (i + 1) for i in range(5))


@pytest.fixture(scope="module")
def L():
    return N.lib()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return set(re.findall(r"^\s*(?:const\s+)?\w+\**\s+\**(\w+)\s*\(", text, flags=re.M))


def test_header_declares_exactly_the_exports():
    assert declared_functions() == set(N.EXPORTS)


def test_library_exports_every_declared_symbol(L):
    out = subprocess.run(["nm", "-D", "--defined-only", N.LIB_PATH], check=True, stdout=subprocess.PIPE,
                         text=True).stdout
    syms = {ln.split()[-1] for ln in out.splitlines() if " T " in ln}
    for name in declared_functions():
        assert name in syms, name
        assert hasattr(L, name)


def test_version_and_status_strings(L):
    assert L.adaln_abi_version() == N.ABI_VERSION == 3
    codes = [N.OK, N.ERR_NULL, N.ERR_SHAPE, N.ERR_DTYPE, N.ERR_ALIGN, N.ERR_ALIAS, N.ERR_TOO_LARGE,
             N.ERR_STRIDE, N.ERR_HIP, N.ERR_ARG]
    names = [N.status_str(c) for c in codes]
    assert len(set(names)) == len(codes)
    assert N.status_str(12345) == "unknown status"


# storage classes the entry points take, as (element stride, row-start alignment in bytes):
# vector loads (16- and 8-byte rows), element gathers (2-byte rows, padded strides), and the
# transposed tiles of tokens-contiguous storage (hidden elements S apart)
LAYOUTS = [(1, 16), (1, 8), (1, 4), (1, 2), (3, 2), (1024, 16), (4096, 2)]
ROW_OPS = (N.OP_LN_MODULATE, N.OP_RESIDUAL_GATE_ADD_LN_MODULATE, N.OP_RMSNORM_SCALE_SHIFT)
HEAD_OPS = (N.OP_QK_HEAD_LAYERNORM, N.OP_QK_RMSNORM)


@pytest.mark.parametrize("D,V", [(4, 4), (8, 8), (12, 4), (512, 8), (2240, 8), (4096, 8), (4100, 4), (8192, 8),
                                 (16392, 8), (65532, 4), (65536, 8)])
def test_order_for_row_ops(D, V):
    for op in ROW_OPS:
        want = None
        for sx_d, align in LAYOUTS:
            o = N.order_for(op, D, sx_d, align)
            d = o.as_dict()
            assert d["V"] == V and d["map"] == N.MAP_INTERLEAVED and d["fold"] == N.FOLD_PAIRWISE, d
            assert d["L"] == 64 * d["W"] and d["W"] >= 1 and (d["W"] & (d["W"] - 1)) == 0, d
            # at most 64 elements per lane: the row is held in registers, read from memory once
            assert 64 * d["L"] >= D, d
            # the order is a function of op and D only: every storage class reduces alike
            want = want or d
            assert d == want, (sx_d, align, d, want)


@pytest.mark.parametrize("D,V", [(4, 4), (12, 4), (64, 8), (128, 8), (132, 4), (256, 8)])
def test_order_for_head_ops(D, V):
    for op in HEAD_OPS:
        for sx_d, align in LAYOUTS:
            assert N.order_for(op, D, sx_d, align).as_dict() == {
                "V": V, "L": 16, "W": 1, "map": N.MAP_INTERLEAVED, "fold": N.FOLD_PAIRWISE}


def test_order_for_rejects(L):
    def rc(op, D, sx_d=1, align=16, out=True):
        import ctypes

        o = N.Order()
        return L.adaln_order_for(op, D, sx_d, align, ctypes.byref(o) if out else None)

    for D in (0, -4, 6, 2242):
        assert rc(N.OP_LN_MODULATE, D) == N.ERR_SHAPE
        assert rc(N.OP_QK_HEAD_LAYERNORM, D) == N.ERR_SHAPE
        with pytest.raises(N.AdalnError):
            N.order_for(N.OP_LN_MODULATE, D)
    assert rc(N.OP_QK_HEAD_LAYERNORM, 260) == N.ERR_SHAPE
    assert rc(N.OP_LN_MODULATE, 65540) == N.ERR_TOO_LARGE
    assert rc(7, 512) == N.ERR_ARG
    assert rc(0, 512) == N.ERR_ARG
    assert rc(N.OP_LN_MODULATE, 512, sx_d=-1) == N.ERR_STRIDE
    for a in (0, 1, 3, 12, -16):
        assert rc(N.OP_LN_MODULATE, 512, align=a) == N.ERR_ALIGN
    assert rc(N.OP_LN_MODULATE, 512, out=False) == N.ERR_NULL


def test_ln_modulate_can_use(L):
    ok = lambda *a: L.ln_modulate_can_use(*a, N.BF16)  # noqa: E731
    assert ok(1, 4096, 4096, 4096 * 4096, 4096, 1, 4096, 4096)
    assert ok(2, 1024, 2240, 2240 * 1024, 1, 1024, 13440, 13440)  # transposed view
    assert ok(0, 0, 4, 0, 0, 1, 0, 0)  # empty
    assert ok(1, 1, 65536, 0, 65536, 1, 0, 0)
    assert not ok(1, 1, 65540, 0, 65540, 1, 0, 0)  # too large
    assert not ok(1, 1, 6, 0, 6, 1, 0, 0)  # D % 4
    assert not ok(1, 1, 0, 0, 0, 1, 0, 0)
    assert not ok(-1, 1, 8, 0, 8, 1, 0, 0)
    assert not ok(1, 2, 8, 16, -8, 1, 0, 0)
    assert not L.ln_modulate_can_use(1, 1, 8, 8, 8, 1, 8, 8, 2)  # dtype


def test_other_can_use(L):
    assert L.residual_gate_add_can_use(1, 4096, 4096, 4096 * 4096, 4096, 4096, 4096 * 4096, 4096, N.BF16)
    assert L.residual_gate_add_can_use(2, 3, 5, 15, 5, 5, 15, 5, N.BF16)  # any D
    assert not L.residual_gate_add_can_use(2, 3, 5, 15, -5, 5, 15, 5, N.BF16)
    assert not L.residual_gate_add_can_use(2, 3, 5, 15, 5, 5, 15, 5, 0)
    assert L.qk_head_layernorm_can_use(1, 4360, 32, 128, 4360 * 4096, 4096, 128, 4360 * 4096, 4096, 128, N.BF16)
    assert L.qk_head_layernorm_can_use(1, 2, 3, 256, 1536, 768, 256, 1536, 768, 256, N.BF16)
    assert not L.qk_head_layernorm_can_use(1, 2, 3, 260, 1560, 780, 260, 1560, 780, 260, N.BF16)
    assert not L.qk_head_layernorm_can_use(1, 2, 3, 126, 756, 378, 126, 756, 378, 126, N.BF16)
    assert L.bias_gelu_tanh_can_use(16384, 12288, 12288, N.BF16)
    assert L.bias_gelu_tanh_can_use(3, 7, 7, N.BF16)
    assert not L.bias_gelu_tanh_can_use(3, 7, -1, N.BF16)
    assert not L.bias_gelu_tanh_can_use(3, 7, 7, 5)


def lnm(L, x=P0, B=1, S=4, D=8, sx=None, scale=P1, ssc=8, shift=P2, ssh=8, eps=1e-6, dtype=N.BF16, out=P3,
        mean=None, rstd=None):
    sx_b, sx_s, sx_d = sx if sx is not None else (S * D, D, 1)
    return L.ln_modulate(x, B, S, D, sx_b, sx_s, sx_d, scale, ssc, shift, ssh, eps, dtype, out, mean, rstd, None)


def test_ln_modulate_rejections(L):
    assert lnm(L, dtype=2) == N.ERR_DTYPE
    assert lnm(L, D=6) == N.ERR_SHAPE
    assert lnm(L, D=0) == N.ERR_SHAPE
    assert lnm(L, B=-1) == N.ERR_SHAPE
    assert lnm(L, D=65540) == N.ERR_TOO_LARGE
    assert lnm(L, sx=(32, -8, 1)) == N.ERR_STRIDE
    assert lnm(L, eps=float("nan")) == N.ERR_ARG
    assert lnm(L, eps=-1.0) == N.ERR_ARG
    assert lnm(L, x=None) == N.ERR_NULL
    assert lnm(L, scale=None) == N.ERR_NULL
    assert lnm(L, out=None) == N.ERR_NULL
    assert lnm(L, x=P0 + 1) == N.ERR_ALIGN
    assert lnm(L, mean=P4 + 2) == N.ERR_ALIGN
    # out overlapping x other than the exact contiguous alias
    assert lnm(L, out=P0 + 16) == N.ERR_ALIAS
    assert lnm(L, out=P0, sx=(64, 16, 1)) == N.ERR_ALIAS  # same base, x not contiguous
    assert lnm(L, out=P1) == N.ERR_ALIAS  # out over scale
    assert lnm(L, out=P2 - 16) == N.ERR_ALIAS  # out tail over shift
    assert lnm(L, mean=P3 + 8) == N.ERR_ALIAS  # stats over out
    assert lnm(L, mean=P4, rstd=P4 + 8) == N.ERR_ALIAS  # mean and rstd overlap
    # an empty problem is a successful no-op even with NULL pointers
    assert lnm(L, x=None, scale=None, shift=None, out=None, B=0) == N.OK
    assert lnm(L, x=None, scale=None, shift=None, out=None, S=0) == N.OK


def lnw(L, ws=P4 + 0x1000000, wsb=1 << 20, **kw):
    """ln_modulate_ws with ln_modulate's arguments (lnm's defaults) and a workspace."""
    a = dict(x=P0, B=1, S=4, D=8, sx=None, scale=P1, ssc=8, shift=P2, ssh=8, eps=1e-6, dtype=N.BF16, out=P3,
             mean=None, rstd=None)
    a.update(kw)
    S, D = a["S"], a["D"]
    sx_b, sx_s, sx_d = a["sx"] if a["sx"] is not None else (S * D, D, 1)
    return L.ln_modulate_ws(a["x"], a["B"], S, D, sx_b, sx_s, sx_d, a["scale"], a["ssc"], a["shift"], a["ssh"],
                            a["eps"], a["dtype"], a["out"], a["mean"], a["rstd"], ws, wsb, None)


def test_ln_modulate_ws_rejections(L):
    # every ln_modulate rejection holds
    assert lnw(L, dtype=2) == N.ERR_DTYPE
    assert lnw(L, D=6) == N.ERR_SHAPE
    assert lnw(L, D=65540) == N.ERR_TOO_LARGE
    assert lnw(L, sx=(32, -8, 1)) == N.ERR_STRIDE
    assert lnw(L, eps=-1.0) == N.ERR_ARG
    assert lnw(L, x=None) == N.ERR_NULL
    assert lnw(L, x=P0 + 1) == N.ERR_ALIGN
    assert lnw(L, out=P0 + 16) == N.ERR_ALIAS
    # the workspace: 16-byte aligned, a non-negative size, overlapping no tensor
    assert lnw(L, ws=P4 + 0x1000008) == N.ERR_ALIGN
    assert lnw(L, wsb=-1) == N.ERR_ARG
    assert lnw(L, ws=P0 - 64, wsb=128) == N.ERR_ALIAS  # over x
    assert lnw(L, ws=P3 + 16, wsb=64) == N.ERR_ALIAS  # over out
    assert lnw(L, ws=P2, wsb=16) == N.ERR_ALIAS  # over shift
    assert lnw(L, ws=P4, wsb=64, mean=P4 + 32) == N.ERR_ALIAS  # over the statistics
    # an empty problem is a successful no-op
    assert lnw(L, x=None, scale=None, shift=None, out=None, B=0) == N.OK


def test_ln_modulate_noalloc_rejections(L):
    def lna(**kw):
        a = dict(x=P0, B=1, S=4, D=8, sx=None, scale=P1, ssc=8, shift=P2, ssh=8, eps=1e-6, dtype=N.BF16, out=P3,
                 mean=None, rstd=None)
        a.update(kw)
        S, D = a["S"], a["D"]
        sx_b, sx_s, sx_d = a["sx"] if a["sx"] is not None else (S * D, D, 1)
        return L.ln_modulate_noalloc(a["x"], a["B"], S, D, sx_b, sx_s, sx_d, a["scale"], a["ssc"], a["shift"],
                                     a["ssh"], a["eps"], a["dtype"], a["out"], a["mean"], a["rstd"], None)

    assert lna(dtype=2) == N.ERR_DTYPE
    assert lna(D=6) == N.ERR_SHAPE
    assert lna(x=None) == N.ERR_NULL
    assert lna(x=P0 + 1) == N.ERR_ALIGN
    assert lna(out=P0 + 16) == N.ERR_ALIAS
    # transposed storage beyond the library's array (1024 groups of 64 tokens), before any HIP call
    assert lna(S=65600, D=8, sx=(8 * 65600, 1, 65600)) == N.ERR_TOO_LARGE
    assert lna(B=2, S=32832, D=8, sx=(8 * 32832, 1, 32832)) == N.ERR_TOO_LARGE
    assert lna(x=None, scale=None, shift=None, out=None, B=0) == N.OK


def test_ln_modulate_workspace_size(L):
    def size(B, S, D, sx=None):
        sx_b, sx_s, sx_d = sx if sx is not None else (D * S, 1, S)  # transposed storage
        return L.ln_modulate_workspace_size(B, S, D, sx_b, sx_s, sx_d)

    group = 64 * 8 * 16 + 64  # 64 tokens x 8 blocks x (mean, m2) words + the group's word, 64-byte slabs
    assert group == 8256
    assert size(2, 1024, 2240) == 32 * group
    assert size(1, 4096, 4096) == 64 * group
    assert size(3, 64, 8) == 3 * group
    assert size(2, 1024, 2240, sx=(2240 * 1088, 1, 1088)) == 32 * group  # padded token rows
    # shapes that never take the workspace path
    assert size(1, 4096, 4096, sx=(4096 * 4096, 4096, 1)) == 0  # contiguous rows
    assert size(2, 96, 512) == 0  # S % 64 != 0
    assert size(1, 128, 516) == 0  # D % 8 != 0
    assert size(1, 64, 4104) == 0  # D > 4096
    assert size(1, 128, 512, sx=(512 * 132, 1, 132)) == 0  # token rows not 16-byte multiples
    assert size(2, 128, 512, sx=(512 * 128 + 4, 1, 128)) == 0  # sample stride not 16-byte multiples
    assert size(0, 64, 512) == 0  # empty
    assert size(1, 64, 6) == 0  # rejected shape
    # tokens within a sample are indexed in 32 bits on that path
    assert size(1, 2**31 - 64, 8) == (2**31 - 64) // 64 * group
    assert size(1, 2**31, 8) == 0


def test_residual_gate_add_rejections(L):
    def rga(res=P0, gate=P1, upd=P2, out=P3, B=2, S=3, D=8, dtype=N.BF16, sr=(24, 8), su=(24, 8), sg=8):
        return L.residual_gate_add(res, sr[0], sr[1], gate, sg, upd, su[0], su[1], B, S, D, dtype, out, None)

    assert rga(dtype=0) == N.ERR_DTYPE
    assert rga(D=-1) == N.ERR_SHAPE
    assert rga(sr=(24, -8)) == N.ERR_STRIDE
    assert rga(res=None) == N.ERR_NULL
    assert rga(gate=P1 + 1) == N.ERR_ALIGN
    assert rga(out=P0 + 2) == N.ERR_ALIAS
    assert rga(out=P2 + 2) == N.ERR_ALIAS
    assert rga(out=P1) == N.ERR_ALIAS
    assert rga(out=P0, sr=(48, 16)) == N.ERR_ALIAS  # exact base but residual not contiguous
    assert rga(res=None, gate=None, upd=None, out=None, B=0) == N.OK
    assert rga(res=None, gate=None, upd=None, out=None, D=0) == N.OK


def test_qk_rejections(L):
    def qk(q=P0, k=P1, wq=P2, bq=P2 + 512, wk=P2 + 1024, bk=P2 + 1536, qo=P3, ko=P4, B=1, S=2, H=3, Dh=128,
           eps=1e-6, dtype=N.BF16):
        sb, ss, sh = S * H * Dh, H * Dh, Dh
        return L.qk_head_layernorm(q, sb, ss, sh, k, sb, ss, sh, B, S, H, Dh, wq, bq, wk, bk, eps, dtype, qo, ko,
                                   None)

    assert qk(dtype=3) == N.ERR_DTYPE
    assert qk(Dh=126) == N.ERR_SHAPE
    assert qk(Dh=260) == N.ERR_TOO_LARGE
    assert qk(eps=float("inf")) == N.ERR_ARG
    assert qk(q=None) == N.ERR_NULL
    assert qk(bq=None) == N.ERR_NULL  # w without b
    assert qk(wk=None, bk=None) == N.ERR_NULL  # affine on one side only
    assert qk(ko=P4 + 1) == N.ERR_ALIGN
    assert qk(qo=P1) == N.ERR_ALIAS  # q_out over k
    assert qk(ko=P3 + 64) == N.ERR_ALIAS  # q_out and k_out overlap
    assert qk(qo=P2 - 64) == N.ERR_ALIAS  # q_out over the weights
    assert qk(q=None, k=None, qo=None, ko=None, S=0) == N.OK


def test_bias_gelu_rejections(L):
    def bg(x=P0, rows=4, width=64, sx=64, bias=P1, dtype=N.BF16, out=P2):
        return L.bias_gelu_tanh(x, rows, width, sx, bias, dtype, out, None)

    assert bg(dtype=0) == N.ERR_DTYPE
    assert bg(rows=-1) == N.ERR_SHAPE
    assert bg(sx=-64) == N.ERR_STRIDE
    assert bg(bias=None) == N.ERR_NULL
    assert bg(out=P2 + 1) == N.ERR_ALIGN
    assert bg(out=P0 + 2) == N.ERR_ALIAS
    assert bg(out=P1 - 2) == N.ERR_ALIAS
    assert bg(out=P0, sx=128) == N.ERR_ALIAS
    assert bg(x=None, bias=None, out=None, rows=0) == N.OK


def test_fused_residual_can_use(L):
    ok = lambda *a: L.residual_gate_add_ln_modulate_can_use(*a, N.BF16)  # noqa: E731
    sq = 4096 * 4096
    assert ok(1, 4096, 4096, sq, 4096, 4096, sq, 4096, 4096, 4096)
    assert ok(4, 4096, 3072, 4096 * 3072, 3072, 6 * 3072, 4096 * 3072, 3072, 6 * 3072, 6 * 3072)
    assert ok(0, 0, 4, 0, 0, 0, 0, 0, 0, 0)
    assert ok(1, 1, 65536, 0, 65536, 0, 0, 65536, 0, 0)
    assert not ok(1, 1, 65540, 0, 65540, 0, 0, 65540, 0, 0)
    assert not ok(1, 1, 6, 0, 6, 0, 0, 6, 0, 0)
    assert not ok(1, 2, 8, 16, 8, 8, 16, 8, -8, 8)
    assert not L.residual_gate_add_ln_modulate_can_use(1, 1, 8, 8, 8, 8, 8, 8, 8, 8, 0)


def test_fused_residual_rejections(L):
    P5, P6, P7 = 0x60000000, 0x70000000, 0x80000000

    def fz(res=P0, gate=P1, upd=P2, scale=P3, shift=P4, ro=P5, out=P6, mean=None, rstd=None, B=2, S=3, D=8,
           eps=1e-6, dtype=N.BF16, sr=(24, 8), su=(24, 8), sg=8, ssc=8, ssh=8):
        return L.residual_gate_add_ln_modulate(res, sr[0], sr[1], gate, sg, upd, su[0], su[1], B, S, D, scale,
                                               ssc, shift, ssh, eps, dtype, ro, out, mean, rstd, None)

    assert fz(dtype=2) == N.ERR_DTYPE
    assert fz(D=6) == N.ERR_SHAPE
    assert fz(D=65540) == N.ERR_TOO_LARGE
    assert fz(su=(24, -8)) == N.ERR_STRIDE
    assert fz(eps=float("nan")) == N.ERR_ARG
    for k in ("res", "gate", "upd", "scale", "shift", "ro", "out"):
        assert fz(**{k: None}) == N.ERR_NULL, k
    assert fz(upd=P2 + 1) == N.ERR_ALIGN
    assert fz(rstd=P7 + 2) == N.ERR_ALIGN
    # allowed: residual_out exactly residual, out exactly update (both contiguous)
    # rejected: any other overlap
    assert fz(ro=P0 + 2) == N.ERR_ALIAS
    assert fz(ro=P0, sr=(48, 16)) == N.ERR_ALIAS  # residual not contiguous
    assert fz(out=P2, su=(48, 16)) == N.ERR_ALIAS  # update not contiguous
    assert fz(ro=P2) == N.ERR_ALIAS  # residual_out over update
    assert fz(out=P0) == N.ERR_ALIAS  # out over residual
    assert fz(out=P5 + 16) == N.ERR_ALIAS  # the two outputs overlap
    assert fz(ro=P1) == N.ERR_ALIAS  # residual_out over gate
    assert fz(out=P3 - 16) == N.ERR_ALIAS  # out tail over scale
    assert fz(mean=P6 + 8) == N.ERR_ALIAS  # stats over out
    assert fz(mean=P7, rstd=P7 + 8) == N.ERR_ALIAS
    assert fz(res=None, gate=None, upd=None, scale=None, shift=None, ro=None, out=None, S=0) == N.OK


def test_rms_can_use(L):
    ok = lambda *a: L.rmsnorm_scale_shift_can_use(*a, N.BF16)  # noqa: E731
    assert ok(1, 4096, 4096, 4096 * 4096, 4096, 1, 4096, 4096)
    assert ok(2, 1024, 2240, 2240 * 1024, 1, 1024, 13440, 13440)
    assert not ok(1, 1, 6, 0, 6, 1, 0, 0)
    assert not ok(1, 1, 65540, 0, 65540, 1, 0, 0)
    assert L.qk_rmsnorm_can_use(1, 4360, 32, 128, 4360 * 4096, 4096, 128, 4360 * 4096, 4096, 128, N.BF16)
    assert not L.qk_rmsnorm_can_use(1, 2, 3, 260, 1560, 780, 260, 1560, 780, 260, N.BF16)
    assert not L.qk_rmsnorm_can_use(1, 2, 3, 128, 768, 384, 128, 768, 384, 128, 0)


def test_rms_rejections(L):
    def rms(x=P0, B=1, S=4, D=8, sx=None, scale=P1, ssc=8, shift=P2, ssh=8, eps=1e-6, dtype=N.BF16, out=P3,
            rinv=None):
        sx_b, sx_s, sx_d = sx if sx is not None else (S * D, D, 1)
        return L.rmsnorm_scale_shift(x, B, S, D, sx_b, sx_s, sx_d, scale, ssc, shift, ssh, eps, dtype, out, rinv,
                                     None)

    assert rms(dtype=0) == N.ERR_DTYPE
    assert rms(D=10) == N.ERR_SHAPE
    assert rms(eps=-1.0) == N.ERR_ARG
    assert rms(shift=None) == N.ERR_NULL
    assert rms(out=P3 + 1) == N.ERR_ALIGN
    assert rms(out=P0 + 16) == N.ERR_ALIAS
    assert rms(rinv=P3 + 8) == N.ERR_ALIAS
    assert rms(x=None, scale=None, shift=None, out=None, B=0) == N.OK

    def qk(q=P0, k=P1, wq=P2, wk=P2 + 1024, qo=P3, ko=P4, B=1, S=2, H=3, Dh=128, eps=1e-6, dtype=N.BF16):
        sb, ss, sh = S * H * Dh, H * Dh, Dh
        return L.qk_rmsnorm(q, sb, ss, sh, k, sb, ss, sh, B, S, H, Dh, wq, wk, eps, dtype, qo, ko, None)

    assert qk(dtype=3) == N.ERR_DTYPE
    assert qk(Dh=126) == N.ERR_SHAPE
    assert qk(eps=float("nan")) == N.ERR_ARG
    assert qk(k=None) == N.ERR_NULL
    assert qk(wk=None) == N.ERR_NULL  # weight on one side only
    assert qk(qo=P1) == N.ERR_ALIAS
    assert qk(ko=P2 + 16) == N.ERR_ALIAS  # k_out over the weights
    assert qk(wq=None, wk=None, qo=P3 + 1) == N.ERR_ALIGN
    assert qk(q=None, k=None, qo=None, ko=None, B=0) == N.OK


def test_modulate_and_temb_can_use(L):
    assert L.modulate_scale_shift_can_use(1, 4096, 4096, 4096 * 4096, 4096, 4096, 0, 4096, 0, N.BF16)
    assert L.modulate_scale_shift_can_use(2, 3, 5, 15, 5, 15, 5, 15, 5, N.BF16)  # per token, any D
    assert not L.modulate_scale_shift_can_use(2, 3, 5, 15, 5, 15, -5, 15, 5, N.BF16)
    assert not L.modulate_scale_shift_can_use(2, 3, 5, 15, 5, 15, 5, 15, 5, N.F32)
    assert L.temb_table_slices_can_use(1, 109120, 6, 3072, 3072, 109120 * 6 * 3072, 6 * 3072, 3072, N.BF16)
    assert L.temb_table_slices_can_use(2, 3, 9, 7, 7, 189, 63, 7, N.F32)
    assert not L.temb_table_slices_can_use(2, 3, 9, 7, 7, 189, 63, 7, 3)
    assert not L.temb_table_slices_can_use(2, -3, 9, 7, 7, 189, 63, 7, N.BF16)


def test_modulate_and_temb_rejections(L):
    def mod(x=P0, scale=P1, shift=P2, out=P3, B=2, S=3, D=8, sx=(24, 8), ssc=(8, 0), ssh=(8, 0), dtype=N.BF16):
        return L.modulate_scale_shift(x, sx[0], sx[1], scale, ssc[0], ssc[1], shift, ssh[0], ssh[1], B, S, D, dtype,
                                      out, None)

    assert mod(dtype=2) == N.ERR_DTYPE
    assert mod(D=-1) == N.ERR_SHAPE
    assert mod(ssc=(8, -1)) == N.ERR_STRIDE
    assert mod(shift=None) == N.ERR_NULL
    assert mod(out=P3 + 1) == N.ERR_ALIGN
    assert mod(out=P0 + 2) == N.ERR_ALIAS
    assert mod(out=P0, sx=(48, 16)) == N.ERR_ALIAS
    assert mod(out=P1 - 4) == N.ERR_ALIAS
    assert mod(x=None, scale=None, shift=None, out=None, S=0) == N.OK

    def temb(table=P0, t=P1, out=P2, B=2, Lq=3, M=6, D=8, st=8, se=(144, 48, 8), dtype=N.BF16):
        return L.temb_table_slices(table, st, t, se[0], se[1], se[2], B, Lq, M, D, dtype, out, None)

    assert temb(dtype=0) == N.ERR_DTYPE
    assert temb(M=-1) == N.ERR_SHAPE
    assert temb(se=(144, -48, 8)) == N.ERR_STRIDE
    assert temb(t=None) == N.ERR_NULL
    assert temb(table=P0 + 2) == N.ERR_ALIGN
    assert temb(t=P1 + 2, dtype=N.F32) == N.ERR_ALIGN
    assert temb(out=P1 + 64) == N.ERR_ALIAS  # out over temb
    assert temb(out=P0 + 4) == N.ERR_ALIAS  # out over the table
    assert temb(table=None, t=None, out=None, M=0) == N.OK


def test_fold_and_fp8_rejections(L):
    P5 = 0x60000000

    assert L.ln_modulate_fold(P0, 1, 4, 6, 24, 6, 1, P1, 6, P2, 6, 1e-6, N.BF16, P3, None, None, None) == N.ERR_SHAPE
    assert L.ln_modulate_fold(P0, 1, 4, 8, 32, 8, 1, P1, 8, P2, 8, 1e-6, N.BF16, P0 + 16, None, None, None) == N.ERR_ALIAS

    def fp8(x=P0, scale=P1, shift=P2, q=P4, out=P3, D=8, S=4, dtype=N.BF16, eps=1e-6, mean=None):
        return L.ln_modulate_fp8(x, 1, S, D, S * D, D, 1, scale, D, shift, D, eps, q, dtype, out, mean, None, None)

    assert fp8(dtype=2) == N.ERR_DTYPE
    assert fp8(D=6) == N.ERR_SHAPE
    assert fp8(eps=float("nan")) == N.ERR_ARG
    assert fp8(q=None) == N.ERR_NULL
    assert fp8(q=P4 + 2) == N.ERR_ALIGN
    assert fp8(out=P3 + 4) == N.ERR_ALIGN  # V = 8: 8-byte aligned rows of bytes
    assert fp8(out=P0) == N.ERR_ALIAS  # an FP8 out may not alias x, not even exactly
    assert fp8(out=P4 - 8) == N.ERR_ALIAS  # out over the scale value
    assert fp8(mean=P5, out=P5 + 8) == N.ERR_ALIAS
    assert fp8(x=None, scale=None, shift=None, q=None, out=None, S=0) == N.OK
