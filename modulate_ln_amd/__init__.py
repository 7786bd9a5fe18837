"""adaLN chain kernels for MI355X (gfx950): a C-ABI library of hand-written HIP
kernels (``libadaln.so``) and this thin torch binding.

    from modulate_ln_amd import ln_modulate, residual_gate_add, qk_head_layernorm, bias_gelu_tanh
    from modulate_ln_amd import residual_gate_add_ln_modulate, rmsnorm_scale_shift, qk_rmsnorm
    from modulate_ln_amd import modulate_scale_shift, temb_table_slices, ln_modulate_fold, ln_modulate_fp8
    from modulate_ln_amd import ln_modulate_workspace, ln_modulate_noalloc  # transposed x

The binding only marshals arguments; torch provides device memory and
streams.  Importing the package does not load the library; the first call
does, and fails loudly if it has not been built.
"""

from ._native import AdalnError, order_for, status_str  # noqa: F401
from .ops import (  # noqa: F401
    bias_gelu_tanh,
    ln_modulate,
    ln_modulate_fold,
    ln_modulate_fp8,
    ln_modulate_noalloc,
    ln_modulate_workspace,
    ln_modulate_workspace_size,
    modulate_scale_shift,
    qk_head_layernorm,
    qk_rmsnorm,
    residual_gate_add,
    residual_gate_add_ln_modulate,
    rmsnorm_scale_shift,
    temb_table_slices,
)

__all__ = [
    "ln_modulate",
    "ln_modulate_workspace",
    "ln_modulate_workspace_size",
    "ln_modulate_noalloc",
    "residual_gate_add",
    "residual_gate_add_ln_modulate",
    "rmsnorm_scale_shift",
    "qk_rmsnorm",
    "modulate_scale_shift",
    "temb_table_slices",
    "ln_modulate_fold",
    "ln_modulate_fp8",
    "qk_head_layernorm",
    "bias_gelu_tanh",
    "order_for",
    "status_str",
    "AdalnError",
]
