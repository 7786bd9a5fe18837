"""ln_modulate_ws (the workspace entry point) through the C ABI: bit-exact with the
oracle's fixed-order fp32 mode and with ln_modulate on the same inputs, on
transposed storage ([B, D, S], tokens contiguous) where the 8 blocks of each
64-token group hand their partial states over through the workspace.

Covered: the Sana transposed workload at full size, hidden sizes from one
vector to 4096 (ragged last steps), padded token and batch strides, more
groups than the resident slots (the persistent loop), one workspace shared
by calls of different shapes in a row, the recompute path (every wait cut to
zero), NaN/Inf rows, and the shapes and sizes that fall back to ln_modulate.
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

from modulate_ln_amd import workloads as W

pytestmark = pytest.mark.gpu

FP32 = 1
DEV = "cuda"


@pytest.fixture(scope="module")
def ops():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import modulate_ln_amd as m

    m._native.lib()  # fail loudly if the library is missing
    return m


def rand_bf16(shape, g, std=1.0, mean=0.0):
    return W.normal(shape, g, mean=mean, std=std)


def bits(t):
    return W.bits(t)


def order(D):
    from modulate_ln_amd import _native as N

    o = N.order_for(N.OP_LN_MODULATE, D)
    return o.V, o.L


def assert_bits_equal(got, want, what=""):
    got, want = np.asarray(got), np.asarray(want)
    assert got.shape == want.shape, (got.shape, want.shape)
    bad = np.argwhere(got != want)
    if bad.size:
        i = tuple(bad[0])
        raise AssertionError("%s: %d mismatches, first at %s: got 0x%04x want 0x%04x" % (
            what, len(bad), i, got[i], want[i]))


def run_ws(ops, x, sc, sh, eps, ws, *, orc=None, what=""):
    """ln_modulate_ws on the (strided) device view x; checked bitwise against ln_modulate
    (output and statistics) and, given the oracle, against its fp32 fixed-order mode."""
    B, S, D = x.shape
    m1 = torch.empty(B * S, dtype=torch.float32, device=DEV)
    r1 = torch.empty(B * S, dtype=torch.float32, device=DEV)
    m0 = torch.empty_like(m1)
    r0 = torch.empty_like(r1)
    y = ops.ln_modulate(x, sc, sh, eps, mean_out=m1, rstd_out=r1, workspace=ws)
    y0 = ops.ln_modulate(x, sc, sh, eps, mean_out=m0, rstd_out=r0)
    torch.cuda.synchronize()
    assert_bits_equal(bits(y.reshape(B * S, D)), bits(y0.reshape(B * S, D)), "ws vs ln_modulate " + what)
    assert torch.equal(m1.view(torch.int32), m0.view(torch.int32)), "mean " + what
    assert torch.equal(r1.view(torch.int32), r0.view(torch.int32)), "rstd " + what
    if orc is not None:
        V, L = order(D)
        want, m32, r32 = orc.ln_modulate(bits(x.contiguous().reshape(B * S, D)), bits(sc.expand(B, D)),
                                         bits(sh.expand(B, D)), S, eps, FP32, V=V, L=L)
        assert_bits_equal(bits(y.reshape(B * S, D)), want, "ws vs oracle " + what)
        assert np.array_equal(m1.cpu().numpy().astype(np.float64), m32), "oracle mean " + what
        assert np.array_equal(r1.cpu().numpy().astype(np.float64), r32), "oracle rstd " + what
    return y


def transposed(B, S, D, g, *, pad_s=0, std=2.0, mean=-0.25):
    """x as the transposed view of [B, D, S + pad_s] storage (tokens contiguous)."""
    xt = rand_bf16((B, D, S + pad_s), g, std=std, mean=mean).to(DEV)
    return xt[:, :, :S].transpose(1, 2)


def test_ws_size_matches_the_view(ops):
    x = torch.empty((2, 2240, 1024), dtype=torch.bfloat16, device=DEV).transpose(1, 2)
    assert ops.ln_modulate_workspace_size(x) == 32 * 8256
    assert ops.ln_modulate_workspace_size(x.contiguous()) == 0


def test_ws_sana_transposed_config(ops, orc):
    wl = W.sana_transposed()
    t = wl.tensors
    x = t["xt"].to(DEV).transpose(1, 2)
    emb = t["emb"].to(DEV)
    ws = ops.ln_modulate_workspace(x)
    for call in range(3):  # the tags advance call by call
        run_ws(ops, x, emb[:, 5], emb[:, 0], wl.meta["eps"], ws, orc=orc if call == 0 else None,
               what="sana transposed, call %d" % call)


@pytest.mark.parametrize("D", [8, 64, 520, 1000, 2240, 3072, 3584, 4096])
@pytest.mark.parametrize("B,S", [(1, 64), (2, 128), (3, 1024)])
def test_ws_transposed_shapes(ops, orc, B, S, D):
    g = torch.Generator().manual_seed(97 * D + S + B)
    x = transposed(B, S, D, g)
    emb = rand_bf16((B, 2, D), g, std=0.1).to(DEV)
    ws = ops.ln_modulate_workspace(x)
    assert ws.numel() == B * S // 64 * 8256
    run_ws(ops, x, emb[:, 1], emb[:, 0], 1e-6, ws, orc=orc, what="B=%d S=%d D=%d" % (B, S, D))


@pytest.mark.parametrize("pad_s", [64, 8])
def test_ws_padded_strides(ops, orc, pad_s):
    """Token rows padded (sx_d = S + pad) and per-sample strides beyond D * S."""
    g = torch.Generator().manual_seed(pad_s)
    B, S, D = 3, 256, 1000
    x = transposed(B, S, D, g, pad_s=pad_s)
    assert x.stride() == (D * (S + pad_s), 1, S + pad_s)
    emb = rand_bf16((B, 2, D), g, std=0.1).to(DEV)
    run_ws(ops, x, emb[:, 1], emb[:, 0], 1e-5, ops.ln_modulate_workspace(x), orc=orc, what="pad %d" % pad_s)


def test_ws_more_groups_than_resident_slots(ops, orc):
    """(4, 4096, 3072): 256 token groups, more than the slots one launch holds at once, so
    the slots loop over groups; every row against the oracle."""
    g = torch.Generator().manual_seed(4096)
    B, S, D = 4, 4096, 3072
    x = transposed(B, S, D, g, std=1.0, mean=0.1)
    emb = rand_bf16((B, 2, D), g, std=0.1).to(DEV)
    run_ws(ops, x, emb[:, 1], emb[:, 0], 1e-6, ops.ln_modulate_workspace(x), orc=orc, what="(4,4096,3072)")


def test_ws_shared_by_shapes_in_a_row(ops):
    """One workspace, large enough for the largest shape, serves calls of different shapes
    one after another: each call leaves it ready for the next."""
    g = torch.Generator().manual_seed(11)
    shapes = [(2, 1024, 2240), (1, 4096, 4096), (1, 64, 8), (3, 512, 520), (2, 1024, 2240), (1, 4096, 4096)]
    xs = {s: transposed(*s, g) for s in set(shapes)}
    embs = {s: rand_bf16((s[0], 2, s[2]), g, std=0.1).to(DEV) for s in set(shapes)}
    ws = ops.ln_modulate_workspace(xs[(1, 4096, 4096)], max(ops.ln_modulate_workspace_size(x) for x in xs.values()))
    for i, s in enumerate(shapes):
        run_ws(ops, xs[s], embs[s][:, 1], embs[s][:, 0], 1e-6, ws, what="call %d shape %s" % (i, s))


def test_ws_recompute_path(ops, orc, monkeypatch):
    """With every wait cut to zero a block recomputes the other blocks' states from x: the
    same bits (and the workspace is still left ready for the next call)."""
    g = torch.Generator().manual_seed(5)
    x = transposed(2, 1024, 2240, g)
    emb = rand_bf16((2, 2, 2240), g, std=0.1).to(DEV)
    ws = ops.ln_modulate_workspace(x)
    monkeypatch.setenv("ADALN_WS_WAIT_US", "0")
    run_ws(ops, x, emb[:, 1], emb[:, 0], 1e-6, ws, orc=orc, what="recompute")
    x2 = transposed(1, 256, 8, g)
    emb2 = rand_bf16((1, 2, 8), g, std=0.1).to(DEV)
    run_ws(ops, x2, emb2[:, 1], emb2[:, 0], 1e-6, ws, orc=orc, what="recompute D=8")
    # the persistent kernel (more groups than one pass of one block per group holds; at
    # D = 4096 the kernel that re-reads its row from LDS) recomputes in the same order
    for shape in ((3, 1024, 2240), (1, 4096, 4096)):
        x3 = transposed(*shape, g)
        emb3 = rand_bf16((shape[0], 2, shape[2]), g, std=0.1).to(DEV)
        run_ws(ops, x3, emb3[:, 1], emb3[:, 0], 1e-6, ops.ln_modulate_workspace(x3), orc=orc,
               what="recompute %s" % (shape,))
    monkeypatch.delenv("ADALN_WS_WAIT_US")
    run_ws(ops, x, emb[:, 1], emb[:, 0], 1e-6, ws, what="after recompute")


def test_ws_non_finite_rows(ops):
    """Rows holding inf or NaN: NaN where ln_modulate has NaN (a NaN's sign is not part of
    the contract, as elsewhere in these suites), the same bits everywhere else."""
    g = torch.Generator().manual_seed(3)
    B, S, D = 1, 128, 2240
    xt = rand_bf16((B, D, S), g).to(DEV)
    xt[0, 17, 3] = float("inf")
    xt[0, 100, 70] = float("nan")
    xt[0, :, 90] = 0
    x = xt.transpose(1, 2)
    emb = rand_bf16((B, 2, D), g, std=0.1).to(DEV)
    y = ops.ln_modulate(x, emb[:, 1], emb[:, 0], 1e-6, workspace=ops.ln_modulate_workspace(x))
    y0 = ops.ln_modulate(x, emb[:, 1], emb[:, 0], 1e-6)
    torch.cuda.synchronize()
    a, b = bits(y.reshape(S, D)), bits(y0.reshape(S, D))
    nan_a, nan_b = (a & 0x7FFF) > 0x7F80, (b & 0x7FFF) > 0x7F80
    assert np.array_equal(nan_a, nan_b)
    assert nan_a[3].all() and nan_a[70].all() and nan_a.sum() == 2 * D  # inf - inf and NaN poison the row
    assert_bits_equal(np.where(nan_a, 0, a), np.where(nan_b, 0, b), "finite rows")
    assert (a[90] == b[90]).all()


def test_ws_fallbacks_are_ln_modulate(ops, orc):
    """Shapes outside the workspace path, and a workspace too small for the shape, run
    ln_modulate's kernels: same bits, the workspace untouched."""
    g = torch.Generator().manual_seed(9)
    cases = [
        rand_bf16((2, 96, 512), g).to(DEV),  # contiguous rows
        transposed(2, 96, 512, g),  # S % 64 != 0
        transposed(1, 128, 516, g),  # D % 8 != 0
        transposed(1, 64, 4104, g),  # D > 4096
    ]
    for x in cases:
        B, S, D = x.shape
        emb = rand_bf16((B, 2, D), g, std=0.1).to(DEV)
        assert ops.ln_modulate_workspace_size(x) == 0
        ws = torch.full((4096,), 0x5A, dtype=torch.uint8, device=DEV)
        run_ws(ops, x, emb[:, 1], emb[:, 0], 1e-6, ws, orc=orc, what="fallback %s %s" % (tuple(x.shape), x.stride()))
        assert bool((ws == 0x5A).all()), "workspace written on a fallback shape"
    x = transposed(2, 1024, 2240, g)
    emb = rand_bf16((2, 2, 2240), g, std=0.1).to(DEV)
    small = torch.full((ops.ln_modulate_workspace_size(x) - 8,), 0x5A, dtype=torch.uint8, device=DEV)
    run_ws(ops, x, emb[:, 1], emb[:, 0], 1e-6, small, what="workspace too small")
    assert bool((small == 0x5A).all()), "too-small workspace written"


def test_ws_broadcast_row_and_no_stats(ops, orc):
    """One adaLN row for every sample (row stride 0), and calls that ask for no statistics."""
    g = torch.Generator().manual_seed(17)
    B, S, D = 3, 1024, 520
    x = transposed(B, S, D, g)
    sc1 = rand_bf16((1, D), g, std=0.1).to(DEV)
    sh1 = rand_bf16((1, D), g, std=0.1).to(DEV)
    sc, sh = sc1.expand(B, D), sh1.expand(B, D)
    assert sc.stride(0) == 0
    ws = ops.ln_modulate_workspace(x)
    run_ws(ops, x, sc, sh, 1e-6, ws, orc=orc, what="broadcast row")
    for shape in ((2, 1024, 2240), (1, 4096, 4096)):
        xs = transposed(*shape, g)
        e = rand_bf16((shape[0], 2, shape[2]), g, std=0.1).to(DEV)
        y = ops.ln_modulate(xs, e[:, 1], e[:, 0], 1e-6, workspace=ops.ln_modulate_workspace(xs))
        y0 = ops.ln_modulate(xs, e[:, 1], e[:, 0], 1e-6)
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16), y0.view(torch.int16)), "no stats %s" % (shape,)


def test_ws_concurrent_streams(ops):
    """Calls on two streams at once, each with a workspace of its own: each grid is sized to
    be resident alone, so together they may not be; a block whose partner is not running
    waits a bounded time and recomputes, so both still give ln_modulate's bits."""
    g = torch.Generator().manual_seed(23)
    shapes = [(2, 1024, 2240), (1, 4096, 4096)]
    xs = [transposed(*s, g) for s in shapes]
    es = [rand_bf16((s[0], 2, s[2]), g, std=0.1).to(DEV) for s in shapes]
    wss = [ops.ln_modulate_workspace(x) for x in xs]
    outs = [torch.empty(s, dtype=torch.bfloat16, device=DEV) for s in shapes]
    want = [ops.ln_modulate(x, e[:, 1], e[:, 0], 1e-6) for x, e in zip(xs, es)]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    torch.cuda.synchronize()
    for rep in range(4):
        for i in range(2):
            with torch.cuda.stream(streams[i]):
                for _ in range(3):
                    ops.ln_modulate(xs[i], es[i][:, 1], es[i][:, 0], 1e-6, out=outs[i], workspace=wss[i])
        torch.cuda.synchronize()
        for i in range(2):
            assert torch.equal(outs[i].view(torch.int16), want[i].view(torch.int16)), "rep %d stream %d" % (rep, i)
