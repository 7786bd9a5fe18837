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


@pytest.mark.parametrize("path", ["workspace", "noalloc"])
def test_graph_workspace_paths(ops, path):
    """ln_modulate_ws (a workspace of the caller's) and ln_modulate_noalloc (the library's
    array) on transposed storage, captured once and replayed on new inputs: each replay
    equals the eager ln_modulate of the inputs it ran on (the hand-over tags advance on the
    device from replay to replay)."""
    g0 = torch.Generator().manual_seed(2024)
    B, S, D = 2, 1024, 2240
    xs = [W.normal((B, D, S), g0, mean=0.1 * i, std=1.0 + i).to(DEV) for i in range(4)]
    emb = W.normal((B, 2, D), g0, std=0.1).to(DEV)
    xt = xs[0].clone()
    x = xt.transpose(1, 2)
    out = torch.empty((B, S, D), dtype=torch.bfloat16, device=DEV)
    ws = ops.ln_modulate_workspace(x) if path == "workspace" else None

    def call():
        if path == "workspace":
            ops.ln_modulate(x, emb[:, 1], emb[:, 0], 1e-6, out=out, workspace=ws)
        else:
            ops.ln_modulate_noalloc(x, emb[:, 1], emb[:, 0], 1e-6, out=out)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up off the default stream, as capture requires
        call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    for rep in range(8):
        xt.copy_(xs[rep % 4])
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        want = ops.ln_modulate(xs[rep % 4].transpose(1, 2), emb[:, 1], emb[:, 0], 1e-6)
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), want.view(torch.int16)), "replay %d" % rep
        call()  # eager work between replays, on the same workspace
        torch.cuda.synchronize()
