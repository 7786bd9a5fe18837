"""Torch-facing binding of the adaLN C ABI: argument marshalling only.

Every function here checks dtypes/devices, allocates outputs with torch when
the caller passes none, reads pointers and strides, and calls the C entry
point of the same name on the current HIP stream.  All arithmetic runs in
the library's kernels.  With ``prepare=True`` a function returns the
marshalled call (a ``Prepared``) instead of issuing it.
"""

from __future__ import annotations

import torch

from . import _native as N


class Prepared:
    """A marshalled call: the C function and its argument tuple, ready to issue.

    Calling it enqueues the kernel(s) again with the same pointers, sizes and
    stream (for tight loops where per-call marshalling would dominate).  It
    holds a reference to every tensor whose address is in its arguments
    (``keep``), so none of them is freed -- and its memory reused by the
    allocator -- while the prepared call exists; the values read are those
    the tensors hold when the call is issued."""

    __slots__ = ("name", "fn", "args", "result", "keep")

    def __init__(self, name, fn, args, result, keep=()):
        self.name, self.fn, self.args, self.result = name, fn, args, result
        self.keep = tuple(t for t in keep if t is not None)

    def __call__(self):
        rc = self.fn(*self.args)
        if rc != N.OK:
            raise N.AdalnError(self.name, rc)
        return self.result


def _stream_handle(t: torch.Tensor, stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream(t.device)
    return int(stream.cuda_stream) if hasattr(stream, "cuda_stream") else int(stream)


def _require(t: torch.Tensor, name: str) -> None:
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if t.dtype != torch.bfloat16:
        raise TypeError("%s must be bfloat16, got %s" % (name, t.dtype))
    if t.device.type != "cuda":
        raise ValueError("%s must be on a HIP device, got %s" % (name, t.device))


def _rows_view(t: torch.Tensor, B: int, D: int, name: str):
    """[B,D] or [B,1,D] adaLN rows -> (tensor, batch stride); element stride must be 1."""
    if t.dim() == 3:
        if t.shape[1] != 1:
            raise ValueError("%s must be [B,1,D] or [B,D], got %s" % (name, tuple(t.shape)))
        t = t[:, 0]
    if t.dim() != 2 or t.shape[1] != D or t.shape[0] not in (B, 1):
        raise ValueError("%s must be [B,D] with B=%d D=%d, got %s" % (name, B, D, tuple(t.shape)))
    if D > 1 and t.stride(1) != 1:
        raise ValueError("%s must have unit stride along the hidden dim" % name)
    sb = t.stride(0) if t.shape[0] == B else 0  # one row broadcast to every sample
    return t, sb


def ln_modulate_workspace_size(x: torch.Tensor) -> int:
    """Bytes of workspace ln_modulate(..., workspace=...) uses for x's shape and strides
    (0 when that shape never takes the workspace path)."""
    if x.dim() != 3:
        raise ValueError("x must be [B,S,D], got %s" % (tuple(x.shape),))
    B, S, D = x.shape
    return int(N.lib().ln_modulate_workspace_size(B, S, D, x.stride(0), x.stride(1), x.stride(2)))


def ln_modulate_workspace(x: torch.Tensor, nbytes: int | None = None) -> torch.Tensor:
    """A zero-filled uint8 workspace on x's device, large enough for x (or nbytes); reuse it
    across calls (the calls leave it ready), one workspace per concurrently running call."""
    n = ln_modulate_workspace_size(x) if nbytes is None else int(nbytes)
    return torch.zeros(max(n, 16), dtype=torch.uint8, device=x.device)


def ln_modulate(x: torch.Tensor, scale: torch.Tensor, shift: torch.Tensor, eps: float = 1e-6, *,
                out: torch.Tensor | None = None, mean_out: torch.Tensor | None = None,
                rstd_out: torch.Tensor | None = None, workspace: torch.Tensor | None = None, stream=None,
                prepare: bool = False):
    """LN(x) * (1 + scale) + shift with every eager bf16 rounding (x: [B,S,D], any strides).
    With `workspace` (from ln_modulate_workspace) the call goes through ln_modulate_ws: the
    same bits, whole-line reads of transposed storage."""
    _require(x, "x")
    _require(scale, "scale")
    _require(shift, "shift")
    if x.dim() != 3:
        raise ValueError("x must be [B,S,D], got %s" % (tuple(x.shape),))
    B, S, D = x.shape
    scale, ssc = _rows_view(scale, B, D, "scale")
    shift, ssh = _rows_view(shift, B, D, "shift")
    if out is None:
        out = torch.empty((B, S, D), dtype=torch.bfloat16, device=x.device)
    else:
        _require(out, "out")
        if tuple(out.shape) != (B, S, D) or not out.is_contiguous():
            raise ValueError("out must be a contiguous [B,S,D] tensor")
    for name, t in (("mean_out", mean_out), ("rstd_out", rstd_out)):
        if t is not None and (t.dtype != torch.float32 or t.numel() != B * S or not t.is_contiguous()
                              or t.device != x.device):
            raise ValueError("%s must be a contiguous float32 tensor of B*S elements on x's device" % name)
    st = _stream_handle(x, stream)
    args = (x.data_ptr(), B, S, D, x.stride(0), x.stride(1), x.stride(2),
            scale.data_ptr(), ssc, shift.data_ptr(), ssh, float(eps), N.BF16, out.data_ptr(),
            mean_out.data_ptr() if mean_out is not None else None,
            rstd_out.data_ptr() if rstd_out is not None else None)
    if workspace is None:
        call = Prepared("ln_modulate", N.lib().ln_modulate, args + (st,), out,
                        keep=(x, scale, shift, out, mean_out, rstd_out))
    else:
        if (not isinstance(workspace, torch.Tensor) or workspace.dtype != torch.uint8
                or not workspace.is_contiguous() or workspace.device != x.device):
            raise ValueError("workspace must be a contiguous uint8 tensor on x's device (ln_modulate_workspace)")
        call = Prepared("ln_modulate_ws", N.lib().ln_modulate_ws,
                        args + (workspace.data_ptr(), workspace.numel(), st), out,
                        keep=(x, scale, shift, out, mean_out, rstd_out, workspace))
    return call if prepare else call()


def ln_modulate_noalloc(x: torch.Tensor, scale: torch.Tensor, shift: torch.Tensor, eps: float = 1e-6, *,
                        out: torch.Tensor, mean_out: torch.Tensor | None = None,
                        rstd_out: torch.Tensor | None = None, stream=None, prepare: bool = False):
    """ln_modulate through ln_modulate_noalloc: the workspace path with the library's own
    device array, for callers that cannot allocate (so `out` must be given).  Calls on one
    device share that array: order them (one stream, or events)."""
    _require(x, "x")
    _require(scale, "scale")
    _require(shift, "shift")
    _require(out, "out")
    if x.dim() != 3:
        raise ValueError("x must be [B,S,D], got %s" % (tuple(x.shape),))
    B, S, D = x.shape
    scale, ssc = _rows_view(scale, B, D, "scale")
    shift, ssh = _rows_view(shift, B, D, "shift")
    if tuple(out.shape) != (B, S, D) or not out.is_contiguous():
        raise ValueError("out must be a contiguous [B,S,D] tensor")
    for name, t in (("mean_out", mean_out), ("rstd_out", rstd_out)):
        if t is not None and (t.dtype != torch.float32 or t.numel() != B * S or not t.is_contiguous()
                              or t.device != x.device):
            raise ValueError("%s must be a contiguous float32 tensor of B*S elements on x's device" % name)
    call = Prepared("ln_modulate_noalloc", N.lib().ln_modulate_noalloc, (
        x.data_ptr(), B, S, D, x.stride(0), x.stride(1), x.stride(2),
        scale.data_ptr(), ssc, shift.data_ptr(), ssh, float(eps), N.BF16, out.data_ptr(),
        mean_out.data_ptr() if mean_out is not None else None,
        rstd_out.data_ptr() if rstd_out is not None else None, _stream_handle(x, stream)), out,
        keep=(x, scale, shift, out, mean_out, rstd_out))
    return call if prepare else call()


def _ln_common(x, scale, shift, out, out_dtype, mean_out, rstd_out):
    _require(x, "x")
    _require(scale, "scale")
    _require(shift, "shift")
    if x.dim() != 3:
        raise ValueError("x must be [B,S,D], got %s" % (tuple(x.shape),))
    B, S, D = x.shape
    scale, ssc = _rows_view(scale, B, D, "scale")
    shift, ssh = _rows_view(shift, B, D, "shift")
    if out is None:
        out = torch.empty((B, S, D), dtype=out_dtype, device=x.device)
    elif out.dtype != out_dtype or tuple(out.shape) != (B, S, D) or not out.is_contiguous():
        raise ValueError("out must be a contiguous %s [B,S,D] tensor" % out_dtype)
    for name, t in (("mean_out", mean_out), ("rstd_out", rstd_out)):
        if t is not None and (t.dtype != torch.float32 or t.numel() != B * S or not t.is_contiguous()
                              or t.device != x.device):
            raise ValueError("%s must be a contiguous float32 tensor of B*S elements on x's device" % name)
    return B, S, D, scale, ssc, shift, ssh, out


def ln_modulate_fold(x: torch.Tensor, scale: torch.Tensor, shift: torch.Tensor, eps: float = 1e-6, *,
                     out: torch.Tensor | None = None, mean_out: torch.Tensor | None = None,
                     rstd_out: torch.Tensor | None = None, stream=None, prepare: bool = False):
    """layer_norm(x, weight=1 + scale, bias=shift) with one rounding: the high-quality-tier fold
    (not the eager chain's bits)."""
    B, S, D, scale, ssc, shift, ssh, out = _ln_common(x, scale, shift, out, torch.bfloat16, mean_out, rstd_out)
    st = _stream_handle(x, stream)
    call = Prepared("ln_modulate_fold", N.lib().ln_modulate_fold, (
        x.data_ptr(), B, S, D, x.stride(0), x.stride(1), x.stride(2),
        scale.data_ptr(), ssc, shift.data_ptr(), ssh, float(eps), N.BF16, out.data_ptr(),
        mean_out.data_ptr() if mean_out is not None else None,
        rstd_out.data_ptr() if rstd_out is not None else None, st), out,
        keep=(x, scale, shift, out, mean_out, rstd_out))
    return call if prepare else call()


def ln_modulate_fp8(x: torch.Tensor, scale: torch.Tensor, shift: torch.Tensor, qscale: torch.Tensor,
                    eps: float = 1e-6, *, out: torch.Tensor | None = None, mean_out: torch.Tensor | None = None,
                    rstd_out: torch.Tensor | None = None, stream=None, prepare: bool = False):
    """ln_modulate's bf16 output quantized to static OCP FP8 E4M3 (torch.float8_e4m3fn) with the
    per-tensor scale qscale (a 1-element float32 device tensor)."""
    if not isinstance(qscale, torch.Tensor) or qscale.dtype != torch.float32 or qscale.numel() != 1 \
            or qscale.device != x.device:
        raise ValueError("qscale must be a 1-element float32 tensor on x's device")
    B, S, D, scale, ssc, shift, ssh, out = _ln_common(x, scale, shift, out, torch.float8_e4m3fn, mean_out,
                                                      rstd_out)
    st = _stream_handle(x, stream)
    call = Prepared("ln_modulate_fp8", N.lib().ln_modulate_fp8, (
        x.data_ptr(), B, S, D, x.stride(0), x.stride(1), x.stride(2),
        scale.data_ptr(), ssc, shift.data_ptr(), ssh, float(eps), qscale.data_ptr(), N.BF16, out.data_ptr(),
        mean_out.data_ptr() if mean_out is not None else None,
        rstd_out.data_ptr() if rstd_out is not None else None, st), out,
        keep=(x, scale, shift, qscale, out, mean_out, rstd_out))
    return call if prepare else call()


def rmsnorm_scale_shift(x: torch.Tensor, scale: torch.Tensor, shift: torch.Tensor, eps: float = 1e-6, *,
                        out: torch.Tensor | None = None, rinv_out: torch.Tensor | None = None, stream=None,
                        prepare: bool = False):
    """RMSNorm(x) * (1 + scale) + shift with every eager bf16 rounding (x: [B,S,D], any strides)."""
    _require(x, "x")
    _require(scale, "scale")
    _require(shift, "shift")
    if x.dim() != 3:
        raise ValueError("x must be [B,S,D], got %s" % (tuple(x.shape),))
    B, S, D = x.shape
    scale, ssc = _rows_view(scale, B, D, "scale")
    shift, ssh = _rows_view(shift, B, D, "shift")
    if out is None:
        out = torch.empty((B, S, D), dtype=torch.bfloat16, device=x.device)
    else:
        _require(out, "out")
        if tuple(out.shape) != (B, S, D) or not out.is_contiguous():
            raise ValueError("out must be a contiguous [B,S,D] tensor")
    if rinv_out is not None and (rinv_out.dtype != torch.float32 or rinv_out.numel() != B * S
                                 or not rinv_out.is_contiguous() or rinv_out.device != x.device):
        raise ValueError("rinv_out must be a contiguous float32 tensor of B*S elements on x's device")
    st = _stream_handle(x, stream)
    call = Prepared("rmsnorm_scale_shift", N.lib().rmsnorm_scale_shift, (
        x.data_ptr(), B, S, D, x.stride(0), x.stride(1), x.stride(2),
        scale.data_ptr(), ssc, shift.data_ptr(), ssh, float(eps), N.BF16, out.data_ptr(),
        rinv_out.data_ptr() if rinv_out is not None else None, st), out, keep=(x, scale, shift, out, rinv_out))
    return call if prepare else call()


def residual_gate_add(residual: torch.Tensor, gate: torch.Tensor, update: torch.Tensor, *,
                      out: torch.Tensor | None = None, stream=None, prepare: bool = False):
    """residual + gate * update with the eager roundings (residual/update [B,S,D], gate [B,D])."""
    _require(residual, "residual")
    _require(gate, "gate")
    _require(update, "update")
    if residual.dim() != 3 or update.shape != residual.shape:
        raise ValueError("residual and update must both be [B,S,D]")
    B, S, D = residual.shape
    gate, sg = _rows_view(gate, B, D, "gate")
    for name, t in (("residual", residual), ("update", update)):
        if D > 1 and t.stride(2) != 1:
            raise ValueError("%s must have unit stride along the hidden dim" % name)
    if out is None:
        out = torch.empty((B, S, D), dtype=torch.bfloat16, device=residual.device)
    else:
        _require(out, "out")
        if tuple(out.shape) != (B, S, D) or not out.is_contiguous():
            raise ValueError("out must be a contiguous [B,S,D] tensor")
    st = _stream_handle(residual, stream)
    call = Prepared("residual_gate_add", N.lib().residual_gate_add, (
        residual.data_ptr(), residual.stride(0), residual.stride(1), gate.data_ptr(), sg,
        update.data_ptr(), update.stride(0), update.stride(1), B, S, D, N.BF16, out.data_ptr(), st), out,
        keep=(residual, gate, update, out))
    return call if prepare else call()


def residual_gate_add_ln_modulate(residual: torch.Tensor, gate: torch.Tensor, update: torch.Tensor,
                                  scale: torch.Tensor, shift: torch.Tensor, eps: float = 1e-6, *,
                                  residual_out: torch.Tensor | None = None, out: torch.Tensor | None = None,
                                  mean_out: torch.Tensor | None = None, rstd_out: torch.Tensor | None = None,
                                  stream=None, prepare: bool = False):
    """(new residual, LN(new residual) * (1 + scale) + shift) with new residual =
    residual + gate * update, every eager bf16 rounding kept; one pass over the rows.

    residual/update [B,S,D] (unit stride along D), gate/scale/shift [B,D] or [B,1,D].
    residual_out may be residual itself and out may be update itself when contiguous."""
    for name, t in (("residual", residual), ("gate", gate), ("update", update), ("scale", scale),
                    ("shift", shift)):
        _require(t, name)
    if residual.dim() != 3 or update.shape != residual.shape:
        raise ValueError("residual and update must both be [B,S,D]")
    B, S, D = residual.shape
    gate, sg = _rows_view(gate, B, D, "gate")
    scale, ssc = _rows_view(scale, B, D, "scale")
    shift, ssh = _rows_view(shift, B, D, "shift")
    for name, t in (("residual", residual), ("update", update)):
        if D > 1 and t.stride(2) != 1:
            raise ValueError("%s must have unit stride along the hidden dim" % name)
    if residual_out is None:
        residual_out = torch.empty((B, S, D), dtype=torch.bfloat16, device=residual.device)
    if out is None:
        out = torch.empty((B, S, D), dtype=torch.bfloat16, device=residual.device)
    for name, t in (("residual_out", residual_out), ("out", out)):
        _require(t, name)
        if tuple(t.shape) != (B, S, D) or not t.is_contiguous():
            raise ValueError("%s must be a contiguous [B,S,D] tensor" % name)
    for name, t in (("mean_out", mean_out), ("rstd_out", rstd_out)):
        if t is not None and (t.dtype != torch.float32 or t.numel() != B * S or not t.is_contiguous()
                              or t.device != residual.device):
            raise ValueError("%s must be a contiguous float32 tensor of B*S elements on residual's device" % name)
    st = _stream_handle(residual, stream)
    call = Prepared("residual_gate_add_ln_modulate", N.lib().residual_gate_add_ln_modulate, (
        residual.data_ptr(), residual.stride(0), residual.stride(1), gate.data_ptr(), sg,
        update.data_ptr(), update.stride(0), update.stride(1), B, S, D,
        scale.data_ptr(), ssc, shift.data_ptr(), ssh, float(eps), N.BF16,
        residual_out.data_ptr(), out.data_ptr(),
        mean_out.data_ptr() if mean_out is not None else None,
        rstd_out.data_ptr() if rstd_out is not None else None, st), (residual_out, out),
        keep=(residual, gate, update, scale, shift, residual_out, out, mean_out, rstd_out))
    return call if prepare else call()


def _affine_rows(t: torch.Tensor, B: int, S: int, D: int, name: str):
    """adaLN rows per sample ([B,D], [B,1,D], broadcast [1,D]) or per token ([B,S,D]) ->
    (tensor, batch stride, token stride); element stride must be 1."""
    if t.dim() == 3 and t.shape[1] == S and S != 1:
        if t.shape[0] not in (B, 1) or t.shape[2] != D:
            raise ValueError("%s must be [B,S,D], [B,1,D] or [B,D], got %s" % (name, tuple(t.shape)))
        if D > 1 and t.stride(2) != 1:
            raise ValueError("%s must have unit stride along the hidden dim" % name)
        return t, (t.stride(0) if t.shape[0] == B else 0), t.stride(1)
    t, sb = _rows_view(t, B, D, name)
    return t, sb, 0


def modulate_scale_shift(x: torch.Tensor, scale: torch.Tensor, shift: torch.Tensor, *,
                         out: torch.Tensor | None = None, stream=None, prepare: bool = False):
    """x * (1 + scale) + shift with the eager roundings; scale/shift one row per sample
    ([B,D] / [B,1,D]) or per token ([B,S,D]); x [B,S,D] with unit stride along D."""
    for name, t in (("x", x), ("scale", scale), ("shift", shift)):
        _require(t, name)
    if x.dim() != 3:
        raise ValueError("x must be [B,S,D]")
    B, S, D = x.shape
    if D > 1 and x.stride(2) != 1:
        raise ValueError("x must have unit stride along the hidden dim")
    scale, ssc_b, ssc_s = _affine_rows(scale, B, S, D, "scale")
    shift, ssh_b, ssh_s = _affine_rows(shift, B, S, D, "shift")
    if out is None:
        out = torch.empty((B, S, D), dtype=torch.bfloat16, device=x.device)
    else:
        _require(out, "out")
        if tuple(out.shape) != (B, S, D) or not out.is_contiguous():
            raise ValueError("out must be a contiguous [B,S,D] tensor")
    st = _stream_handle(x, stream)
    call = Prepared("modulate_scale_shift", N.lib().modulate_scale_shift, (
        x.data_ptr(), x.stride(0), x.stride(1), scale.data_ptr(), ssc_b, ssc_s, shift.data_ptr(), ssh_b, ssh_s,
        B, S, D, N.BF16, out.data_ptr(), st), out, keep=(x, scale, shift, out))
    return call if prepare else call()


def temb_table_slices(table: torch.Tensor, temb: torch.Tensor, *, out: torch.Tensor | None = None, stream=None,
                      prepare: bool = False):
    """The nmod slices of table + temb.float() in one pass: table fp32 [nmod, D] (or with leading
    singleton dims), temb bf16/fp32 [B, L, nmod, D] (unit stride along D).  Returns an fp32
    tensor [nmod, B, L, D]; out[m] is slice m, contiguous."""
    if not isinstance(table, torch.Tensor) or not isinstance(temb, torch.Tensor):
        raise TypeError("table and temb must be torch.Tensors")
    if table.dtype != torch.float32:
        raise TypeError("table must be float32, got %s" % table.dtype)
    if temb.dtype not in (torch.bfloat16, torch.float32):
        raise TypeError("temb must be bfloat16 or float32, got %s" % temb.dtype)
    for name, t in (("table", table), ("temb", temb)):
        if t.device.type != "cuda":
            raise ValueError("%s must be on a HIP device" % name)
    if temb.dim() != 4:
        raise ValueError("temb must be [B, L, nmod, D]")
    B, L, M, D = temb.shape
    table = table.reshape(-1, table.shape[-1]) if table.dim() > 2 else table
    if table.dim() != 2 or tuple(table.shape) != (M, D):
        raise ValueError("table must be [nmod, D] = [%d, %d]" % (M, D))
    for name, t in (("table", table), ("temb", temb)):
        if D > 1 and t.stride(-1) != 1:
            raise ValueError("%s must have unit stride along D" % name)
    if out is None:
        out = torch.empty((M, B, L, D), dtype=torch.float32, device=temb.device)
    elif out.dtype != torch.float32 or tuple(out.shape) != (M, B, L, D) or not out.is_contiguous():
        raise ValueError("out must be a contiguous float32 [nmod, B, L, D] tensor")
    dt = N.F32 if temb.dtype == torch.float32 else N.BF16
    st = _stream_handle(temb, stream)
    call = Prepared("temb_table_slices", N.lib().temb_table_slices, (
        table.data_ptr(), table.stride(0), temb.data_ptr(), temb.stride(0), temb.stride(1), temb.stride(2),
        B, L, M, D, dt, out.data_ptr(), st), out, keep=(table, temb, out))
    return call if prepare else call()


def qk_head_layernorm(q: torch.Tensor, k: torch.Tensor, wq: torch.Tensor | None = None,
                      bq: torch.Tensor | None = None, wk: torch.Tensor | None = None,
                      bk: torch.Tensor | None = None, eps: float = 1e-6, *,
                      q_out: torch.Tensor | None = None, k_out: torch.Tensor | None = None, stream=None,
                      prepare: bool = False):
    """Per-head affine LayerNorm of q and k ([B,S,H,Dh] each) in one launch."""
    _require(q, "q")
    _require(k, "k")
    if q.dim() != 4 or k.shape != q.shape:
        raise ValueError("q and k must both be [B,S,H,Dh]")
    B, S, H, Dh = q.shape
    for name, t in (("q", q), ("k", k)):
        if Dh > 1 and t.stride(3) != 1:
            raise ValueError("%s must have unit stride along head_dim" % name)
    ws = (wq, bq, wk, bk)
    if any(w is None for w in ws) and not all(w is None for w in ws):
        raise ValueError("wq, bq, wk, bk go together (all or none)")
    for name, w in zip(("wq", "bq", "wk", "bk"), ws):
        if w is not None:
            _require(w, name)
            if w.numel() != Dh or not w.is_contiguous():
                raise ValueError("%s must be a contiguous [Dh] tensor" % name)
    if q_out is None:
        q_out = torch.empty((B, S, H, Dh), dtype=torch.bfloat16, device=q.device)
    if k_out is None:
        k_out = torch.empty((B, S, H, Dh), dtype=torch.bfloat16, device=q.device)
    for name, t in (("q_out", q_out), ("k_out", k_out)):
        _require(t, name)
        if tuple(t.shape) != (B, S, H, Dh) or not t.is_contiguous():
            raise ValueError("%s must be a contiguous [B,S,H,Dh] tensor" % name)
    ptr = lambda t: t.data_ptr() if t is not None else None  # noqa: E731
    st = _stream_handle(q, stream)
    call = Prepared("qk_head_layernorm", N.lib().qk_head_layernorm, (
        q.data_ptr(), q.stride(0), q.stride(1), q.stride(2),
        k.data_ptr(), k.stride(0), k.stride(1), k.stride(2),
        B, S, H, Dh, ptr(wq), ptr(bq), ptr(wk), ptr(bk), float(eps), N.BF16,
        q_out.data_ptr(), k_out.data_ptr(), st), (q_out, k_out), keep=(q, k, wq, bq, wk, bk, q_out, k_out))
    return call if prepare else call()


def qk_rmsnorm(q: torch.Tensor, k: torch.Tensor, wq: torch.Tensor | None = None, wk: torch.Tensor | None = None,
               eps: float = 1e-6, *, q_out: torch.Tensor | None = None, k_out: torch.Tensor | None = None,
               stream=None, prepare: bool = False):
    """Per-head RMSNorm of q and k ([B,S,H,Dh] each) with optional weights, one launch."""
    _require(q, "q")
    _require(k, "k")
    if q.dim() != 4 or k.shape != q.shape:
        raise ValueError("q and k must both be [B,S,H,Dh]")
    B, S, H, Dh = q.shape
    for name, t in (("q", q), ("k", k)):
        if Dh > 1 and t.stride(3) != 1:
            raise ValueError("%s must have unit stride along head_dim" % name)
    if (wq is None) != (wk is None):
        raise ValueError("wq and wk go together (both or none)")
    for name, w in (("wq", wq), ("wk", wk)):
        if w is not None:
            _require(w, name)
            if w.numel() != Dh or not w.is_contiguous():
                raise ValueError("%s must be a contiguous [Dh] tensor" % name)
    if q_out is None:
        q_out = torch.empty((B, S, H, Dh), dtype=torch.bfloat16, device=q.device)
    if k_out is None:
        k_out = torch.empty((B, S, H, Dh), dtype=torch.bfloat16, device=q.device)
    for name, t in (("q_out", q_out), ("k_out", k_out)):
        _require(t, name)
        if tuple(t.shape) != (B, S, H, Dh) or not t.is_contiguous():
            raise ValueError("%s must be a contiguous [B,S,H,Dh] tensor" % name)
    ptr = lambda t: t.data_ptr() if t is not None else None  # noqa: E731
    st = _stream_handle(q, stream)
    call = Prepared("qk_rmsnorm", N.lib().qk_rmsnorm, (
        q.data_ptr(), q.stride(0), q.stride(1), q.stride(2),
        k.data_ptr(), k.stride(0), k.stride(1), k.stride(2),
        B, S, H, Dh, ptr(wq), ptr(wk), float(eps), N.BF16, q_out.data_ptr(), k_out.data_ptr(), st), (q_out, k_out),
        keep=(q, k, wq, wk, q_out, k_out))
    return call if prepare else call()


def bias_gelu_tanh(x: torch.Tensor, bias: torch.Tensor, *, out: torch.Tensor | None = None,
                   stream=None, prepare: bool = False):
    """bf16(gelu_tanh(bf16(x + bias))) for x [rows, width] (unit stride along width)."""
    _require(x, "x")
    _require(bias, "bias")
    if x.dim() != 2:
        raise ValueError("x must be [rows, width]")
    rows, width = x.shape
    if bias.numel() != width or not bias.is_contiguous():
        raise ValueError("bias must be a contiguous [width] tensor")
    if width > 1 and x.stride(1) != 1:
        raise ValueError("x must have unit stride along width")
    if out is None:
        out = torch.empty((rows, width), dtype=torch.bfloat16, device=x.device)
    else:
        _require(out, "out")
        if tuple(out.shape) != (rows, width) or not out.is_contiguous():
            raise ValueError("out must be a contiguous [rows, width] tensor")
    st = _stream_handle(x, stream)
    call = Prepared("bias_gelu_tanh", N.lib().bias_gelu_tanh,
                    (x.data_ptr(), rows, width, x.stride(0), bias.data_ptr(), N.BF16, out.data_ptr(), st), out,
        keep=(x, bias, out))
    return call if prepare else call()
