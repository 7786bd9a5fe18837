"""Seeded synthetic inputs for the adaLN chain.

This module only draws random numbers and lays them out; it holds none of
the chain's arithmetic.  Both the HIP path's callers (tests, benchmark) and
the oracle's callers use it, so that the two sides see identical inputs.

Recipe (every config): a CPU ``torch.Generator`` seeded with ``seed``; draws
happen in the order listed; each draw is fp32 ``randn`` (or ``rand``),
scaled and shifted in fp32, then rounded once to bf16 (torch's CPU
round-to-nearest-even).  The shapes and value scales are the ones the pages
test and profile on: Sana 1024px (2, 1024, 2240) with transposed
activations and an nmod=6 adaLN split, GLM-Image (1, 4096, 4096) and the
(1, 4360, 32, 128) q/k heads, and a 20-block DiT chain at hidden 3072.
"""

from __future__ import annotations

from dataclasses import dataclass, field

import torch


def _gen(seed: int) -> torch.Generator:
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    return g


def normal(shape, g: torch.Generator, mean: float = 0.0, std: float = 1.0) -> torch.Tensor:
    """fp32 N(mean, std^2) draw, rounded once to bf16."""
    t = torch.randn(*shape, generator=g, dtype=torch.float32)
    if std != 1.0:
        t = t * std
    if mean != 0.0:
        t = t + mean
    return t.to(torch.bfloat16)


@dataclass
class Workload:
    name: str
    tensors: dict = field(default_factory=dict)
    meta: dict = field(default_factory=dict)


def ln_small(seed: int = 0) -> Workload:
    """x [1,256,512] ~N(0,1); scale, shift [1,512] ~N(0,0.1); eps 1e-6; contiguous."""
    g = _gen(seed)
    x = normal((1, 256, 512), g)
    scale = normal((1, 512), g, std=0.1)
    shift = normal((1, 512), g, std=0.1)
    return Workload("ln_modulate (1,256,512)", dict(x=x, scale=scale, shift=shift), dict(eps=1e-6))


def sana_transposed(seed: int = 0, B: int = 2, S: int = 1024, D: int = 2240, nmod: int = 6) -> Workload:
    """Sana 1024px: x logical [B,S,D] stored as [B,D,S] (a transposed view).

    xt [B,D,S] ~N(0,1) then x = xt.transpose(1, 2); emb [B,nmod,D] ~N(0,0.1);
    shift = emb[:,0], scale = emb[:,nmod-1], gate = emb[:,2 % nmod] (views with
    batch stride nmod*D); eps 1e-6.
    """
    g = _gen(seed)
    xt = normal((B, D, S), g)
    emb = normal((B, nmod, D), g, std=0.1)
    x = xt.transpose(1, 2)
    return Workload(
        "ln_modulate (%d,%d,%d) transposed" % (B, S, D),
        dict(x=x, xt=xt, emb=emb, shift=emb[:, 0], scale=emb[:, nmod - 1], gate=emb[:, 2 % nmod]),
        dict(eps=1e-6, nmod=nmod),
    )


def glm_square(seed: int = 0, B: int = 1, S: int = 4096, D: int = 4096, outlier_p: float = 0.01,
               outlier_scale: float = 20.0) -> Workload:
    """GLM-Image (1,4096,4096): x ~N(0,1) with 1% outliers x20; scale, shift,
    gate [B,D] ~N(0,0.1); update ~N(0,1); eps 1e-5.

    Draw order: x (fp32), outlier mask (rand < p), scale, shift, gate, update.
    The outliers are applied in fp32 before the single bf16 rounding.
    """
    g = _gen(seed)
    x32 = torch.randn(B, S, D, generator=g, dtype=torch.float32)
    mask = torch.rand(B, S, D, generator=g, dtype=torch.float32) < outlier_p
    x32 = torch.where(mask, x32 * outlier_scale, x32)
    x = x32.to(torch.bfloat16)
    del x32, mask
    scale = normal((B, D), g, std=0.1)
    shift = normal((B, D), g, std=0.1)
    gate = normal((B, D), g, std=0.1)
    update = normal((B, S, D), g)
    return Workload("ln_modulate + residual_gate_add (%d,%d,%d)" % (B, S, D),
                    dict(x=x, scale=scale, shift=shift, gate=gate, update=update), dict(eps=1e-5))


def glm_qk(seed: int = 0, B: int = 1, S: int = 4360, H: int = 32, Dh: int = 128) -> Workload:
    """q, k [B,S,H,Dh] ~N(0,1); wq, wk ~N(1,0.05); bq, bk ~N(0,0.02); eps 1e-6.

    Draw order: q, k, wq, bq, wk, bk.
    """
    g = _gen(seed)
    q = normal((B, S, H, Dh), g)
    k = normal((B, S, H, Dh), g)
    wq = normal((Dh,), g, mean=1.0, std=0.05)
    bq = normal((Dh,), g, std=0.02)
    wk = normal((Dh,), g, mean=1.0, std=0.05)
    bk = normal((Dh,), g, std=0.02)
    return Workload("qk_head_layernorm (%d,%d,%d,%d)" % (B, S, H, Dh),
                    dict(q=q, k=k, wq=wq, bq=bq, wk=wk, bk=bk), dict(eps=1e-6))


def dit_chain(seed: int = 0, B: int = 4, S: int = 4096, D: int = 3072, blocks: int = 20) -> Workload:
    """20-block DiT chain on x [4,4096,3072] ~N(0,1); per block emb [B,6,D] ~N(0,0.1).

    Per block k the six adaLN rows are (shift1, scale1, gate1, shift2, scale2,
    gate2) = emb_k[:,0..5].  Draw order: x, emb_0, ..., emb_{blocks-1}.
    """
    g = _gen(seed)
    x = normal((B, S, D), g)
    embs = [normal((B, 6, D), g, std=0.1) for _ in range(blocks)]
    return Workload("DiT chain %d blocks (%d,%d,%d)" % (blocks, B, S, D), dict(x=x, embs=embs),
                    dict(eps=1e-6, blocks=blocks))


def wan_bias_gelu(seed: int = 0, rows: int = 4 * 4096, width: int = 12288) -> Workload:
    """x [rows, width] ~N(0,1); bias [width] ~N(0,0.1).  Draw order: x, bias."""
    g = _gen(seed)
    x = normal((rows, width), g)
    bias = normal((width,), g, std=0.1)
    return Workload("bias_gelu_tanh (%d,%d)" % (rows, width), dict(x=x, bias=bias), {})


def wan_temb(seed: int = 0, B: int = 1, frames: int = 31, tokens_per_frame: int = 44 * 80, nmod: int = 6,
             D: int = 3072) -> Workload:
    """The adaLN table and per-token timestep embedding of a Wan-style DiT at 704x1280, 121
    frames: 31 latent frames of 44x80 tokens (109,120 tokens), 6 slices, hidden 3072 -- the
    size at which the eager (table + temb.float()) holds about 8 GB of fp32.

    table fp32 [nmod, D] ~N(0, 0.1); temb_frame bf16 [B, tokens_per_frame, nmod, D] ~N(0, 1),
    one latent frame's tokens.  Draw order: table, temb_frame.  The full temb is temb_frame
    repeated along the token axis `frames` times (meta["frames"]): tile(temb_frame, frames)."""
    g = _gen(seed)
    table = torch.randn((nmod, D), generator=g, dtype=torch.float32) * 0.1
    temb_frame = normal((B, tokens_per_frame, nmod, D), g)
    return Workload("temb_table_slices (%d,%d,%d,%d)" % (B, frames * tokens_per_frame, nmod, D),
                    dict(table=table, temb_frame=temb_frame), dict(frames=frames))


def tile(t: torch.Tensor, frames: int) -> torch.Tensor:
    """t [B, T, ...] -> [B, frames*T, ...]: the block repeated along axis 1 (works on any device)."""
    return t.repeat(1, frames, *([1] * (t.dim() - 2)))


def bits(t: torch.Tensor):
    """bf16 tensor -> numpy uint16 bit patterns in logical row-major order (a copy)."""
    import numpy as np

    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def from_bits(a) -> torch.Tensor:
    """numpy uint16 bit patterns -> CPU bf16 tensor."""
    import numpy as np

    a = np.ascontiguousarray(a, dtype=np.uint16)
    return torch.from_numpy(a.view(np.int16).copy()).view(torch.bfloat16)
