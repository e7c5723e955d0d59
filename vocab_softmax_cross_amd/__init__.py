"""Fused large-vocabulary softmax cross-entropy for MI355X (gfx950).

The computation lives in ``libvsce.so`` (HIP kernels behind the C ABI of
``include/vsce.h``); this package binds it (``_lib``, same names as the C
ABI), exposes it to PyTorch (``functional``) and builds it (``build``).
"""
from .functional import (
    FusedCrossEntropy,
    LinearCrossEntropy,
    SplitCrossEntropy,
    backward_from_stats,
    cross_entropy,
    flce_forward_backward,
    gemm_bf16_nt,
    linear_cross_entropy,
    forward_fused_inplace,
    forward_stats,
    scale_grad,
    status,
)

__all__ = [
    "cross_entropy",
    "linear_cross_entropy",
    "flce_forward_backward",
    "gemm_bf16_nt",
    "forward_fused_inplace",
    "forward_stats",
    "backward_from_stats",
    "scale_grad",
    "status",
    "FusedCrossEntropy",
    "SplitCrossEntropy",
    "LinearCrossEntropy",
]
