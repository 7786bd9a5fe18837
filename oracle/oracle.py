"""Python view of the CPU oracle (``adaln_oracle.c``).

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, by ``__graft_entry__.smoke``
and by the CPU-baseline leg of ``bench.py``.  The product package never
imports it, and it never imports the product package.

Tensors cross this boundary as numpy ``uint16`` arrays holding bf16 bit
patterns (row-major, logical layout).  Modes:

* ``FP64`` -- the plain two-pass double definition of LayerNorm, every later
  step in double and rounded once to bf16;
* ``FP32`` -- the fp32 Welford algorithm in the fixed (V, L) order described
  at the top of ``adaln_oracle.c``, every later step in fp32 with a bf16
  rounding at each eager op boundary.
"""

from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

FP64 = 0
FP32 = 1

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "adaln_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

_lib = None


GCC_FLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off", "-fno-fast-math",
             "-fopenmp", "-Wall", "-Wextra"]


def compile_source(src: str, out: str) -> str:
    """gcc a C oracle source into a shared library (plain IEEE fp32: no contraction, no fast-math)."""
    tmp = out + ".tmp%d" % os.getpid()
    subprocess.run(["gcc", *GCC_FLAGS, "-o", tmp, src, "-lm"], check=True)
    os.replace(tmp, out)
    return out


def build(force: bool = True) -> str:
    """Compile the oracle (always when force, else only if the source is newer)."""
    if not force and os.path.exists(_LIB) and os.path.getmtime(_LIB) >= os.path.getmtime(_SRC):
        return _LIB
    return compile_source(_SRC, _LIB)


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        build()
    _lib = load_library(_LIB)
    return _lib


def load_library(path: str):
    """Load a compiled oracle library and declare its signatures."""
    lib = ctypes.CDLL(path)
    u16p = ctypes.POINTER(ctypes.c_uint16)
    f32p = ctypes.POINTER(ctypes.c_float)
    f64p = ctypes.POINTER(ctypes.c_double)
    i64 = ctypes.c_int64
    lib.orc_f32_from_bf16.argtypes = [ctypes.c_uint16]
    lib.orc_f32_from_bf16.restype = ctypes.c_float
    lib.orc_bf16_from_f32.argtypes = [ctypes.c_float]
    lib.orc_bf16_from_f32.restype = ctypes.c_uint16
    lib.orc_bf16_from_f64.argtypes = [ctypes.c_double]
    lib.orc_bf16_from_f64.restype = ctypes.c_uint16
    lib.orc_bf16_from_f32_array.argtypes = [f32p, u16p, i64]
    lib.orc_bf16_from_f64_array.argtypes = [f64p, u16p, i64]
    lib.orc_welford_seq.argtypes = [f32p, i64, f32p, f32p]
    lib.orc_welford_combine.argtypes = [f32p, f32p, f32p]
    lib.orc_layernorm_stats.argtypes = [u16p, i64, i64, ctypes.c_float, ctypes.c_int, ctypes.c_int,
                                        ctypes.c_int, f64p, f64p]
    lib.orc_ln_modulate.argtypes = [u16p, i64, i64, i64, u16p, u16p, ctypes.c_float, ctypes.c_int,
                                    ctypes.c_int, ctypes.c_int, u16p, f64p, f64p]
    lib.orc_residual_gate_add.argtypes = [u16p, u16p, u16p, i64, i64, i64, ctypes.c_int, u16p]
    lib.orc_residual_gate_add_ln_modulate.argtypes = [u16p, u16p, u16p, i64, i64, i64, u16p, u16p,
                                                      ctypes.c_float, ctypes.c_int, ctypes.c_int,
                                                      ctypes.c_int, u16p, u16p, f64p, f64p]
    lib.orc_qk_head_layernorm.argtypes = [u16p, i64, i64, u16p, u16p, ctypes.c_float, ctypes.c_int,
                                          ctypes.c_int, ctypes.c_int, u16p]
    lib.orc_rmsnorm_scale_shift.argtypes = [u16p, i64, i64, i64, u16p, u16p, ctypes.c_float, ctypes.c_int,
                                            ctypes.c_int, ctypes.c_int, u16p, f64p]
    lib.orc_qk_rmsnorm.argtypes = [u16p, i64, i64, u16p, ctypes.c_float, ctypes.c_int, ctypes.c_int,
                                   ctypes.c_int, u16p]
    lib.orc_modulate_scale_shift.argtypes = [u16p, i64, i64, i64, u16p, i64, i64, u16p, i64, i64, ctypes.c_int,
                                             u16p]
    lib.orc_temb_table_slices.argtypes = [f32p, ctypes.c_void_p, ctypes.c_int, i64, i64, i64, i64, f32p]
    u8p = ctypes.POINTER(ctypes.c_uint8)
    lib.orc_f64_from_fp8e4m3.argtypes = [ctypes.c_uint8]
    lib.orc_f64_from_fp8e4m3.restype = ctypes.c_double
    lib.orc_fp8e4m3_from_f32.argtypes = [ctypes.c_float]
    lib.orc_fp8e4m3_from_f32.restype = ctypes.c_uint8
    lib.orc_fp8e4m3_from_f64.argtypes = [ctypes.c_double]
    lib.orc_fp8e4m3_from_f64.restype = ctypes.c_uint8
    lib.orc_fp8e4m3_from_f32_array.argtypes = [f32p, u8p, i64]
    lib.orc_ln_modulate_fold.argtypes = [u16p, i64, i64, i64, u16p, u16p, ctypes.c_float, ctypes.c_int,
                                         ctypes.c_int, ctypes.c_int, u16p, f64p, f64p]
    lib.orc_ln_modulate_fp8.argtypes = [u16p, i64, i64, i64, u16p, u16p, ctypes.c_float, ctypes.c_float,
                                        ctypes.c_int, ctypes.c_int, ctypes.c_int, u8p, f64p, f64p]
    lib.orc_set_threads.argtypes = [ctypes.c_int]
    lib.orc_set_threads.restype = None
    lib.orc_get_threads.argtypes = []
    lib.orc_get_threads.restype = ctypes.c_int
    lib.orc_gelu_tanh_f64.argtypes = [ctypes.c_double]
    lib.orc_gelu_tanh_f64.restype = ctypes.c_double
    lib.orc_bias_gelu_tanh.argtypes = [u16p, i64, i64, u16p, u16p, f64p]
    for name in ("orc_layernorm_stats", "orc_ln_modulate", "orc_residual_gate_add",
                 "orc_qk_head_layernorm", "orc_bias_gelu_tanh"):
        getattr(lib, name).restype = ctypes.c_int
    return lib


def _u16(a) -> np.ndarray:
    a = np.ascontiguousarray(a)
    if a.dtype != np.uint16:
        raise TypeError("expected bf16 bit patterns as uint16, got %s" % a.dtype)
    return a


def _p(a, ctype):
    return a.ctypes.data_as(ctypes.POINTER(ctype))


def _check(rc: int, name: str) -> None:
    if rc != 0:
        raise ValueError("oracle %s rejected its arguments (rc=%d)" % (name, rc))


# --- bf16 conversions -------------------------------------------------------

def bf16_from_f32(a) -> np.ndarray:
    a = np.ascontiguousarray(a, dtype=np.float32)
    out = np.empty(a.shape, dtype=np.uint16)
    _load().orc_bf16_from_f32_array(_p(a, ctypes.c_float), _p(out, ctypes.c_uint16), a.size)
    return out


def bf16_from_f64(a) -> np.ndarray:
    a = np.ascontiguousarray(a, dtype=np.float64)
    out = np.empty(a.shape, dtype=np.uint16)
    _load().orc_bf16_from_f64_array(_p(a, ctypes.c_double), _p(out, ctypes.c_uint16), a.size)
    return out


def f32_from_bf16(bits) -> np.ndarray:
    """Widen bf16 bit patterns to float32 (exact: the bits become the upper half)."""
    b = _u16(bits)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


# --- Welford primitives (for the oracle's own pins) ------------------------

def welford_seq(x) -> tuple:
    x = np.ascontiguousarray(x, dtype=np.float32)
    m = ctypes.c_float()
    m2 = ctypes.c_float()
    _load().orc_welford_seq(_p(x, ctypes.c_float), x.size, ctypes.byref(m), ctypes.byref(m2))
    return np.float32(m.value), np.float32(m2.value)


def welford_combine(a, b) -> tuple:
    a = np.ascontiguousarray(a, dtype=np.float32)
    b = np.ascontiguousarray(b, dtype=np.float32)
    out = np.empty(3, dtype=np.float32)
    _load().orc_welford_combine(_p(a, ctypes.c_float), _p(b, ctypes.c_float), _p(out, ctypes.c_float))
    return tuple(np.float32(v) for v in out)


# --- the chain's operations --------------------------------------------------

def layernorm_stats(x, eps: float, mode: int, V: int = 8, L: int = 64):
    """Per-row (mean, rstd) of x [R, D] (bf16 bits)."""
    x = _u16(x)
    R, D = x.shape
    mean = np.empty(R, dtype=np.float64)
    rstd = np.empty(R, dtype=np.float64)
    rc = _load().orc_layernorm_stats(_p(x, ctypes.c_uint16), R, D, eps, mode, V, L,
                                     _p(mean, ctypes.c_double), _p(rstd, ctypes.c_double))
    _check(rc, "layernorm_stats")
    return mean, rstd


def ln_modulate(x, scale, shift, S: int, eps: float, mode: int, V: int = 8, L: int = 64):
    """out = bf16 chain of LN(x)*(1+scale)+shift.

    x [B*S, D], scale/shift [B, D] (bf16 bits).  Returns (out bits [B*S, D],
    mean [B*S] float64, rstd [B*S] float64).
    """
    x, scale, shift = _u16(x), _u16(scale), _u16(shift)
    R, D = x.shape
    B = scale.shape[0]
    if R != B * S or scale.shape != (B, D) or shift.shape != (B, D):
        raise ValueError("shape mismatch")
    out = np.empty((R, D), dtype=np.uint16)
    mean = np.empty(R, dtype=np.float64)
    rstd = np.empty(R, dtype=np.float64)
    rc = _load().orc_ln_modulate(_p(x, ctypes.c_uint16), B, S, D, _p(scale, ctypes.c_uint16),
                                 _p(shift, ctypes.c_uint16), eps, mode, V, L, _p(out, ctypes.c_uint16),
                                 _p(mean, ctypes.c_double), _p(rstd, ctypes.c_double))
    _check(rc, "ln_modulate")
    return out, mean, rstd


def residual_gate_add(res, gate, upd, S: int, mode: int = FP32):
    """out = bf16(res + bf16(gate*upd)); res/upd [B*S, D], gate [B, D] (bf16 bits)."""
    res, gate, upd = _u16(res), _u16(gate), _u16(upd)
    R, D = res.shape
    B = gate.shape[0]
    if R != B * S or upd.shape != (R, D) or gate.shape != (B, D):
        raise ValueError("shape mismatch")
    out = np.empty((R, D), dtype=np.uint16)
    rc = _load().orc_residual_gate_add(_p(res, ctypes.c_uint16), _p(gate, ctypes.c_uint16),
                                       _p(upd, ctypes.c_uint16), B, S, D, mode, _p(out, ctypes.c_uint16))
    _check(rc, "residual_gate_add")
    return out


def rmsnorm_scale_shift(x, scale, shift, S: int, eps: float, mode: int, V: int = 8, L: int = 64):
    """out = bf16 chain of RMSNorm(x)*(1+scale)+shift.

    x [B*S, D], scale/shift [B, D] (bf16 bits).  Returns (out bits [B*S, D],
    rinv [B*S] float64: 1/sqrt(mean(x^2)+eps)).
    """
    x, scale, shift = _u16(x), _u16(scale), _u16(shift)
    R, D = x.shape
    B = scale.shape[0]
    if R != B * S or scale.shape != (B, D) or shift.shape != (B, D):
        raise ValueError("shape mismatch")
    out = np.empty((R, D), dtype=np.uint16)
    rinv = np.empty(R, dtype=np.float64)
    rc = _load().orc_rmsnorm_scale_shift(_p(x, ctypes.c_uint16), B, S, D, _p(scale, ctypes.c_uint16),
                                         _p(shift, ctypes.c_uint16), eps, mode, V, L, _p(out, ctypes.c_uint16),
                                         _p(rinv, ctypes.c_double))
    _check(rc, "rmsnorm_scale_shift")
    return out, rinv


def qk_rmsnorm(x, w, eps: float, mode: int, V: int = 8, L: int = 16):
    """RMSNorm of each head row with an optional weight.  x [R, Dh]; w [Dh] or None."""
    x = _u16(x)
    R, Dh = x.shape
    if w is not None:
        w = _u16(w)
        if w.shape != (Dh,):
            raise ValueError("shape mismatch")
    out = np.empty((R, Dh), dtype=np.uint16)
    rc = _load().orc_qk_rmsnorm(_p(x, ctypes.c_uint16), R, Dh, _p(w, ctypes.c_uint16) if w is not None else None,
                                eps, mode, V, L, _p(out, ctypes.c_uint16))
    _check(rc, "qk_rmsnorm")
    return out


def modulate_scale_shift(x, scale, shift, S: int, mode: int = FP32):
    """out = bf16 chain of x*(1+scale)+shift.  x [B*S, D]; scale/shift [B, D] (one row per
    sample) or [B*S, D] (one row per token), bf16 bits."""
    x, scale, shift = _u16(x), _u16(scale), _u16(shift)
    R, D = x.shape
    B = R // S if S else 0

    def strides(t):
        if t.shape == (R, D):
            return S * D, D
        if t.shape[1] == D and t.shape[0] == B:
            return D, 0
        raise ValueError("scale/shift must be [B, D] or [B*S, D]")

    ssc, ssh = strides(scale), strides(shift)
    out = np.empty((R, D), dtype=np.uint16)
    rc = _load().orc_modulate_scale_shift(_p(x, ctypes.c_uint16), B, S, D, _p(scale, ctypes.c_uint16), ssc[0],
                                          ssc[1], _p(shift, ctypes.c_uint16), ssh[0], ssh[1], mode,
                                          _p(out, ctypes.c_uint16))
    _check(rc, "modulate_scale_shift")
    return out


def temb_table_slices(table, temb, temb_is_f32: bool = False):
    """table fp32 [nmod, D]; temb [B, L, nmod, D] (bf16 bits as uint16, or float32) ->
    out fp32 [nmod, B, L, D] with out[m] = table[m] + temb[:, :, m] in fp32."""
    table = np.ascontiguousarray(table, dtype=np.float32)
    nmod, D = table.shape
    if temb_is_f32:
        temb = np.ascontiguousarray(temb, dtype=np.float32)
    else:
        temb = _u16(temb)
    B, L, m2, D2 = temb.shape
    if (m2, D2) != (nmod, D):
        raise ValueError("shape mismatch")
    out = np.empty((nmod, B, L, D), dtype=np.float32)
    rc = _load().orc_temb_table_slices(_p(table, ctypes.c_float), temb.ctypes.data_as(ctypes.c_void_p),
                                       1 if temb_is_f32 else 0, B, L, nmod, D, _p(out, ctypes.c_float))
    _check(rc, "temb_table_slices")
    return out


def fp8_from_f32(a) -> np.ndarray:
    """float32 array -> OCP e4m3 codes (uint8), nearest with ties to even."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    out = np.empty(a.shape, dtype=np.uint8)
    _load().orc_fp8e4m3_from_f32_array(_p(a, ctypes.c_float), _p(out, ctypes.c_uint8), a.size)
    return out


def f64_from_fp8(codes) -> np.ndarray:
    """OCP e4m3 codes -> their values as float64."""
    c = np.ascontiguousarray(codes, dtype=np.uint8)
    lib = _load()
    return np.array([lib.orc_f64_from_fp8e4m3(int(v)) for v in c.ravel()], dtype=np.float64).reshape(c.shape)


def ln_modulate_fold(x, scale, shift, S: int, eps: float, mode: int, V: int = 8, L: int = 64):
    """Single-rounding fold: bf16(fma(bf16(1+scale), (x-mean)*rstd, shift)).  Returns
    (out bits, mean, rstd) like ln_modulate."""
    x, scale, shift = _u16(x), _u16(scale), _u16(shift)
    R, D = x.shape
    B = scale.shape[0]
    if R != B * S or scale.shape != (B, D) or shift.shape != (B, D):
        raise ValueError("shape mismatch")
    out = np.empty((R, D), dtype=np.uint16)
    mean = np.empty(R, dtype=np.float64)
    rstd = np.empty(R, dtype=np.float64)
    rc = _load().orc_ln_modulate_fold(_p(x, ctypes.c_uint16), B, S, D, _p(scale, ctypes.c_uint16),
                                      _p(shift, ctypes.c_uint16), eps, mode, V, L, _p(out, ctypes.c_uint16),
                                      _p(mean, ctypes.c_double), _p(rstd, ctypes.c_double))
    _check(rc, "ln_modulate_fold")
    return out, mean, rstd


def ln_modulate_fp8(x, scale, shift, S: int, eps: float, qscale: float, mode: int, V: int = 8, L: int = 64):
    """ln_modulate's bf16 output quantized to static OCP e4m3 with per-tensor scale qscale.
    Returns (codes uint8 [B*S, D], mean, rstd)."""
    x, scale, shift = _u16(x), _u16(scale), _u16(shift)
    R, D = x.shape
    B = scale.shape[0]
    if R != B * S or scale.shape != (B, D) or shift.shape != (B, D):
        raise ValueError("shape mismatch")
    out = np.empty((R, D), dtype=np.uint8)
    mean = np.empty(R, dtype=np.float64)
    rstd = np.empty(R, dtype=np.float64)
    rc = _load().orc_ln_modulate_fp8(_p(x, ctypes.c_uint16), B, S, D, _p(scale, ctypes.c_uint16),
                                     _p(shift, ctypes.c_uint16), eps, qscale, mode, V, L, _p(out, ctypes.c_uint8),
                                     _p(mean, ctypes.c_double), _p(rstd, ctypes.c_double))
    _check(rc, "ln_modulate_fp8")
    return out, mean, rstd


def residual_gate_add_ln_modulate(res, gate, upd, scale, shift, S: int, eps: float, mode: int,
                                  V: int = 8, L: int = 64):
    """res_out = bf16(res + bf16(gate*upd)), out = ln_modulate(res_out, scale, shift).

    res/upd [B*S, D], gate/scale/shift [B, D] (bf16 bits).  Returns
    (res_out bits, out bits, mean [B*S] float64, rstd [B*S] float64).
    """
    res, gate, upd, scale, shift = _u16(res), _u16(gate), _u16(upd), _u16(scale), _u16(shift)
    R, D = res.shape
    B = gate.shape[0]
    if R != B * S or upd.shape != (R, D) or any(t.shape != (B, D) for t in (gate, scale, shift)):
        raise ValueError("shape mismatch")
    res_out = np.empty((R, D), dtype=np.uint16)
    out = np.empty((R, D), dtype=np.uint16)
    mean = np.empty(R, dtype=np.float64)
    rstd = np.empty(R, dtype=np.float64)
    rc = _load().orc_residual_gate_add_ln_modulate(
        _p(res, ctypes.c_uint16), _p(gate, ctypes.c_uint16), _p(upd, ctypes.c_uint16), B, S, D,
        _p(scale, ctypes.c_uint16), _p(shift, ctypes.c_uint16), eps, mode, V, L,
        _p(res_out, ctypes.c_uint16), _p(out, ctypes.c_uint16), _p(mean, ctypes.c_double),
        _p(rstd, ctypes.c_double))
    _check(rc, "residual_gate_add_ln_modulate")
    return res_out, out, mean, rstd


def qk_head_layernorm(x, w, b, eps: float, mode: int, V: int = 8, L: int = 16):
    """Affine LayerNorm of each head row.  x [R, Dh]; w, b [Dh] or both None."""
    x = _u16(x)
    R, Dh = x.shape
    out = np.empty((R, Dh), dtype=np.uint16)
    if (w is None) != (b is None):
        raise ValueError("w and b go together")
    wp = _p(_u16(w), ctypes.c_uint16) if w is not None else None
    bp = _p(_u16(b), ctypes.c_uint16) if b is not None else None
    if w is not None:
        w, b = _u16(w), _u16(b)
        wp, bp = _p(w, ctypes.c_uint16), _p(b, ctypes.c_uint16)
    rc = _load().orc_qk_head_layernorm(_p(x, ctypes.c_uint16), R, Dh, wp, bp, eps, mode, V, L,
                                       _p(out, ctypes.c_uint16))
    _check(rc, "qk_head_layernorm")
    return out


def gelu_tanh_f64(z: float) -> float:
    return _load().orc_gelu_tanh_f64(float(z))


def bias_gelu_tanh(x, bias):
    """z = bf16(x+bias); out = bf16(gelu_tanh(z)) in double.  Returns (out bits, value f64)."""
    x, bias = _u16(x), _u16(bias)
    rows, width = x.shape
    out = np.empty((rows, width), dtype=np.uint16)
    val = np.empty((rows, width), dtype=np.float64)
    rc = _load().orc_bias_gelu_tanh(_p(x, ctypes.c_uint16), rows, width, _p(bias, ctypes.c_uint16),
                                    _p(out, ctypes.c_uint16), _p(val, ctypes.c_double))
    _check(rc, "bias_gelu_tanh")
    return out, val


def set_threads(n: int) -> None:
    """OpenMP threads of the row loops (results are independent of it)."""
    _load().orc_set_threads(int(n))


def get_threads() -> int:
    return int(_load().orc_get_threads())
