"""ln_modulate_noalloc through the C ABI: the allocation-free variant of ln_modulate_ws
(its workspace a fixed array inside the library), checked bit for bit against
ln_modulate_ws with a workspace of the caller's on two calls in a row, the
second with a smaller input, plus the size limit and a shape that needs no
workspace.  Collected last: it shares the library's array with nothing else.
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

from modulate_ln_amd import workloads as W

pytestmark = pytest.mark.gpu

DEV = "cuda"
FP32 = 1


@pytest.fixture(scope="module")
def N():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from modulate_ln_amd import _native as N

    N.lib()  # fail loudly if the library is missing
    return N


def transposed(B, S, D, g):
    return W.normal((B, D, S), g, mean=-0.25, std=2.0).to(DEV).transpose(1, 2)


def args(x, sc, sh, out, mean, rstd):
    B, S, D = x.shape
    return (x.data_ptr(), B, S, D, x.stride(0), x.stride(1), x.stride(2), sc.data_ptr(), sc.stride(0),
            sh.data_ptr(), sh.stride(0), 1e-6, 1, out.data_ptr(), mean.data_ptr(), rstd.data_ptr())


def both(N, x, sc, sh):
    """(out, mean, rstd) of ln_modulate_noalloc and of ln_modulate_ws on the same inputs."""
    B, S, D = x.shape
    res = []
    for fn in ("noalloc", "ws"):
        out = torch.full((B, S, D), float("nan"), dtype=torch.bfloat16, device=DEV)
        mean = torch.full((B * S,), float("nan"), dtype=torch.float32, device=DEV)
        rstd = torch.full((B * S,), float("nan"), dtype=torch.float32, device=DEV)
        stream = torch.cuda.current_stream().cuda_stream
        if fn == "noalloc":
            rc = N.lib().ln_modulate_noalloc(*args(x, sc, sh, out, mean, rstd), stream)
        else:
            nb = N.lib().ln_modulate_workspace_size(B, S, D, x.stride(0), x.stride(1), x.stride(2))
            ws = torch.zeros(max(nb, 16), dtype=torch.uint8, device=DEV)
            rc = N.lib().ln_modulate_ws(*args(x, sc, sh, out, mean, rstd), ws.data_ptr(), nb, stream)
        assert rc == N.OK, N.status_str(rc)
        torch.cuda.synchronize()
        res.append((out, mean, rstd))
    return res


def assert_same(a, b, what):
    for u, v, name in zip(a, b, ("out", "mean", "rstd")):
        iu, iv = u.view(torch.int16 if u.dtype == torch.bfloat16 else torch.int32), \
            v.view(torch.int16 if v.dtype == torch.bfloat16 else torch.int32)
        bad = int((iu != iv).sum())
        assert bad == 0, "%s %s: %d elements differ" % (what, name, bad)


def test_noalloc_matches_ws_two_calls_second_smaller(N, orc):
    g = torch.Generator().manual_seed(2240)
    x1 = transposed(2, 1024, 2240, g)  # 32 groups of 64 tokens
    e1 = W.normal((2, 2, 2240), g, std=0.1).to(DEV)
    x2 = transposed(1, 256, 1000, g)  # 4 groups, a ragged last vector step
    e2 = W.normal((1, 2, 1000), g, std=0.1).to(DEV)
    for i, (x, e) in enumerate(((x1, e1), (x2, e2))):
        got, want = both(N, x, e[:, 1], e[:, 0])
        assert_same(got, want, "call %d %s" % (i, tuple(x.shape)))
        assert not torch.isnan(got[0]).any()
    # and the first call's output against the oracle's fixed-order fp32 mode
    B, S, D = x1.shape
    o = N.order_for(N.OP_LN_MODULATE, D)
    want, _, _ = orc.ln_modulate(W.bits(x1.contiguous().reshape(B * S, D)), W.bits(e1[:, 1]), W.bits(e1[:, 0]),
                                 S, 1e-6, FP32, V=o.V, L=o.L)
    got, _ = both(N, x1, e1[:, 1], e1[:, 0])
    assert np.array_equal(W.bits(got[0].reshape(B * S, D)), want)


def test_noalloc_shape_without_workspace(N):
    """Contiguous rows take ln_modulate's kernels: no array, same bits."""
    g = torch.Generator().manual_seed(1)
    x = W.normal((2, 100, 3072), g).to(DEV)
    e = W.normal((2, 2, 3072), g, std=0.1).to(DEV)
    got, want = both(N, x, e[:, 1], e[:, 0])
    assert_same(got, want, "contiguous")


def test_noalloc_rejects_beyond_its_array(N):
    """65536 tokens fit the library's array, 65600 do not: ADALN_ERR_TOO_LARGE, nothing launched."""
    g = torch.Generator().manual_seed(2)
    D = 8
    for S, rc_want in ((65600, N.ERR_TOO_LARGE), (65536, N.OK)):
        x = transposed(1, S, D, g)
        e = W.normal((1, 2, D), g, std=0.1).to(DEV)
        out = torch.zeros((1, S, D), dtype=torch.bfloat16, device=DEV)
        m = torch.zeros(S, dtype=torch.float32, device=DEV)
        r = torch.zeros(S, dtype=torch.float32, device=DEV)
        rc = N.lib().ln_modulate_noalloc(*args(x, e[:, 1], e[:, 0], out, m, r),
                                         torch.cuda.current_stream().cuda_stream)
        torch.cuda.synchronize()
        assert rc == rc_want, (S, N.status_str(rc))
        if rc_want != N.OK:
            assert not out.any(), "a rejected call wrote its output"
        else:  # the largest size the array holds: 1024 groups, the same bits as ln_modulate
            import modulate_ln_amd as ops

            m0 = torch.empty_like(m)
            r0 = torch.empty_like(r)
            want = ops.ln_modulate(x, e[:, 1], e[:, 0], 1e-6, mean_out=m0, rstd_out=r0)
            torch.cuda.synchronize()
            assert torch.equal(out.view(torch.int16), want.view(torch.int16))
            assert torch.equal(m.view(torch.int32), m0.view(torch.int32))
            assert torch.equal(r.view(torch.int32), r0.view(torch.int32))
