"""The adaLN kernels under HIP graph capture (torch.cuda.CUDAGraph): the fused
20-block DiT chain, captured once, replayed several times with eager work and
synchronizations between the replays; every replay must equal the eager run
bit for bit.  The library launches plain kernels only (no memset or copy
nodes), so a captured chain is just its kernel launches."""

from __future__ import annotations

import pytest
import torch

from modulate_ln_amd import workloads as W

from test_gpu_parity import DEV

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ops():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import modulate_ln_amd as m

    m._native.lib()
    return m


def chain(ops, x, h, embs, eps):
    """one ln_modulate, 2*blocks - 1 fused residual + ln_modulate calls, one gate-add; in place on x, h"""
    e0 = embs[0]
    ops.ln_modulate(x, e0[:, 1], e0[:, 0], eps, out=h)
    for i, emb in enumerate(embs):
        ops.residual_gate_add_ln_modulate(x, emb[:, 2], h, emb[:, 4], emb[:, 3], eps, residual_out=x, out=h)
        if i + 1 < len(embs):
            nxt = embs[i + 1]
            ops.residual_gate_add_ln_modulate(x, emb[:, 5], h, nxt[:, 1], nxt[:, 0], eps, residual_out=x, out=h)
        else:
            ops.residual_gate_add(x, emb[:, 5], h, out=x)


@pytest.mark.parametrize("shape", [(1, 512, 3072, 4), (2, 64, 2240, 3)])
def test_graph_replays_equal_eager(ops, shape):
    B, S, D, blocks = shape
    wl = W.dit_chain(B=B, S=S, D=D, blocks=blocks)
    eps = wl.meta["eps"]
    x0 = wl.tensors["x"].to(DEV)
    embs = [e.to(DEV) for e in wl.tensors["embs"]]
    xe, he = x0.clone(), torch.empty_like(x0)
    chain(ops, xe, he, embs, eps)
    torch.cuda.synchronize()

    x, h = x0.clone(), torch.empty_like(x0)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up off the default stream, as capture requires
        chain(ops, x, h, embs, eps)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        chain(ops, x, h, embs, eps)
    for rep in range(4):
        x.copy_(x0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(x.view(torch.int16), xe.view(torch.int16)), "replay %d" % rep
        assert torch.equal(h.view(torch.int16), he.view(torch.int16)), "replay %d" % rep
        ops.ln_modulate(x0, embs[0][:, 1], embs[0][:, 0], eps)  # eager work between replays
        torch.cuda.synchronize()
