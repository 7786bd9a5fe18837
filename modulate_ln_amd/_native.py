"""ctypes view of ``libadaln.so`` (built in-tree by ``modulate_ln_amd.build``).

Loading fails loudly when the library is missing: there is no fallback
implementation of any operation in this package.
"""

from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libadaln.so")

# status codes and constants (include/adaln.h)
OK = 0
ERR_NULL = -1
ERR_SHAPE = -2
ERR_DTYPE = -3
ERR_ALIGN = -4
ERR_ALIAS = -5
ERR_TOO_LARGE = -6
ERR_STRIDE = -7
ERR_HIP = -8
ERR_ARG = -9
BF16 = 1
F32 = 2
OP_LN_MODULATE = 1
OP_QK_HEAD_LAYERNORM = 2
OP_RESIDUAL_GATE_ADD_LN_MODULATE = 3
OP_RMSNORM_SCALE_SHIFT = 4
OP_QK_RMSNORM = 5
MAP_INTERLEAVED = 1
FOLD_PAIRWISE = 1
ABI_VERSION = 3

# every symbol include/adaln.h declares
EXPORTS = (
    "ln_modulate",
    "ln_modulate_can_use",
    "ln_modulate_ws",
    "ln_modulate_workspace_size",
    "ln_modulate_noalloc",
    "residual_gate_add",
    "residual_gate_add_can_use",
    "qk_head_layernorm",
    "qk_head_layernorm_can_use",
    "bias_gelu_tanh",
    "bias_gelu_tanh_can_use",
    "residual_gate_add_ln_modulate",
    "residual_gate_add_ln_modulate_can_use",
    "rmsnorm_scale_shift",
    "rmsnorm_scale_shift_can_use",
    "qk_rmsnorm",
    "qk_rmsnorm_can_use",
    "modulate_scale_shift",
    "modulate_scale_shift_can_use",
    "temb_table_slices",
    "temb_table_slices_can_use",
    "ln_modulate_fold",
    "ln_modulate_fp8",
    "adaln_order_for",
    "adaln_status_str",
    "adaln_abi_version",
)

_lib = None


class AdalnError(RuntimeError):
    """A non-zero status from the C ABI."""

    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__("%s failed: %s (status %d)" % (fn, status_str(status), status))


def lib():
    """The loaded library (loaded once)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            "libadaln.so is not built at %s; run `python -m modulate_ln_amd.build` "
            "(or __graft_entry__.build())" % LIB_PATH
        )
    L = ctypes.CDLL(LIB_PATH)
    vp, i64, f32, ci = ctypes.c_void_p, ctypes.c_int64, ctypes.c_float, ctypes.c_int
    L.ln_modulate.argtypes = [vp, i64, i64, i64, i64, i64, i64, vp, i64, vp, i64, f32, ci, vp, vp, vp, vp]
    L.ln_modulate_can_use.argtypes = [i64, i64, i64, i64, i64, i64, i64, i64, ci]
    L.ln_modulate_ws.argtypes = [vp, i64, i64, i64, i64, i64, i64, vp, i64, vp, i64, f32, ci, vp, vp, vp, vp, i64,
                                 vp]
    L.ln_modulate_workspace_size.argtypes = [i64, i64, i64, i64, i64, i64]
    L.ln_modulate_noalloc.argtypes = [vp, i64, i64, i64, i64, i64, i64, vp, i64, vp, i64, f32, ci, vp, vp, vp, vp]
    L.residual_gate_add.argtypes = [vp, i64, i64, vp, i64, vp, i64, i64, i64, i64, i64, ci, vp, vp]
    L.residual_gate_add_can_use.argtypes = [i64, i64, i64, i64, i64, i64, i64, i64, ci]
    L.qk_head_layernorm.argtypes = [vp, i64, i64, i64, vp, i64, i64, i64, i64, i64, i64, i64,
                                    vp, vp, vp, vp, f32, ci, vp, vp, vp]
    L.qk_head_layernorm_can_use.argtypes = [i64, i64, i64, i64, i64, i64, i64, i64, i64, i64, ci]
    L.bias_gelu_tanh.argtypes = [vp, i64, i64, i64, vp, ci, vp, vp]
    L.bias_gelu_tanh_can_use.argtypes = [i64, i64, i64, ci]
    L.residual_gate_add_ln_modulate.argtypes = [vp, i64, i64, vp, i64, vp, i64, i64, i64, i64, i64,
                                                vp, i64, vp, i64, f32, ci, vp, vp, vp, vp, vp]
    L.residual_gate_add_ln_modulate_can_use.argtypes = [i64, i64, i64, i64, i64, i64, i64, i64, i64,
                                                        i64, ci]
    L.rmsnorm_scale_shift.argtypes = [vp, i64, i64, i64, i64, i64, i64, vp, i64, vp, i64, f32, ci, vp, vp, vp]
    L.rmsnorm_scale_shift_can_use.argtypes = [i64, i64, i64, i64, i64, i64, i64, i64, ci]
    L.qk_rmsnorm.argtypes = [vp, i64, i64, i64, vp, i64, i64, i64, i64, i64, i64, i64, vp, vp, f32, ci, vp, vp,
                             vp]
    L.qk_rmsnorm_can_use.argtypes = [i64, i64, i64, i64, i64, i64, i64, i64, i64, i64, ci]
    L.modulate_scale_shift.argtypes = [vp, i64, i64, vp, i64, i64, vp, i64, i64, i64, i64, i64, ci, vp, vp]
    L.modulate_scale_shift_can_use.argtypes = [i64, i64, i64, i64, i64, i64, i64, i64, i64, ci]
    L.temb_table_slices.argtypes = [vp, i64, vp, i64, i64, i64, i64, i64, i64, i64, ci, vp, vp]
    L.temb_table_slices_can_use.argtypes = [i64, i64, i64, i64, i64, i64, i64, i64, ci]
    L.ln_modulate_fold.argtypes = [vp, i64, i64, i64, i64, i64, i64, vp, i64, vp, i64, f32, ci, vp, vp, vp, vp]
    L.ln_modulate_fp8.argtypes = [vp, i64, i64, i64, i64, i64, i64, vp, i64, vp, i64, f32, vp, ci, vp, vp, vp,
                                  vp]
    L.adaln_order_for.argtypes = [ci, i64, i64, ci, ctypes.POINTER(Order)]
    L.adaln_status_str.argtypes = [ci]
    L.adaln_status_str.restype = ctypes.c_char_p
    L.adaln_abi_version.argtypes = []
    for name in EXPORTS:
        if name != "adaln_status_str":
            getattr(L, name).restype = ci
    L.ln_modulate_workspace_size.restype = i64
    if L.adaln_abi_version() != ABI_VERSION:
        raise ImportError("libadaln.so ABI version %d, binding expects %d" % (L.adaln_abi_version(), ABI_VERSION))
    _lib = L
    return L


def status_str(status: int) -> str:
    return lib().adaln_status_str(int(status)).decode()


def check(fn: str, status: int) -> None:
    if status != OK:
        raise AdalnError(fn, status)


class Order(ctypes.Structure):
    """adaln_order: the fixed fp32 reduction order of a row (include/adaln.h)."""

    _fields_ = [("V", ctypes.c_int), ("L", ctypes.c_int), ("W", ctypes.c_int), ("map", ctypes.c_int),
                ("fold", ctypes.c_int)]

    def as_dict(self):
        return {f: getattr(self, f) for f, _ in self._fields_}


def order_for(op: int, D: int, sx_d: int = 1, align_bytes: int = 16) -> Order:
    """The library's fixed fp32 reduction order for a row of D elements of op stored with
    element stride sx_d and row starts aligned to align_bytes (V, L, W, map, fold)."""
    o = Order()
    check("adaln_order_for", lib().adaln_order_for(op, D, sx_d, align_bytes, ctypes.byref(o)))
    return o
