"""ctypes binding of libvsce.so: the C ABI of include/vsce.h under the same names.

Argument marshalling only: every function here forwards plain device pointers,
sizes and a HIP stream handle to the library and raises if the library
returns an error code.  There is no fallback: without the built library (on
the host or the GPU) importing the functions raises.
"""
from __future__ import annotations

import ctypes
import os
from ctypes import c_float, c_int32, c_int64, c_size_t, c_uint32, c_void_p

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libvsce.so")

# vsce_dtype, vsce_reduction and return codes (include/vsce.h)
F32, BF16, F16 = 0, 1, 2
REDUCTION_NONE, REDUCTION_MEAN, REDUCTION_SUM = 0, 1, 2
REDUCTIONS = {"none": REDUCTION_NONE, "mean": REDUCTION_MEAN, "sum": REDUCTION_SUM}
OK, ERR_INVALID, ERR_UNSUPPORTED, ERR_LAUNCH, ERR_TOO_LARGE = 0, -1, -2, -3, -4
NOALLOC_MAX_ROWS = 65536
STATUS_BAD_TARGET = 1
STATS_STRIDE = 4
PARTIAL_STRIDE = 8
FLAG_LONG_ROWS_RING = 1
WS_W, WS_SUM_W, WS_N_VALID, WS_N_INVALID, WS_STATUS, WS_HEADER_BYTES = 0, 8, 16, 24, 32, 256
WS_INV_W, WS_INV_N_VALID = 40, 44

EXPORTS = ("vsce_workspace_bytes", "ce_forward_fused_inplace", "ce_forward_fused_inplace_timed",
           "ce_forward_fused_inplace_noalloc",
           "ce_forward_stats", "ce_forward_stats_partial", "ce_merge_stats",
           "ce_backward_from_stats", "ce_scale_grad", "vsce_gemm_bf16_nt", "vsce_gemm_bf16",
           "vsce_flce_workspace_bytes", "flce_forward_backward", "vsce_strerror", "vsce_version")
GEMM_OUT_BF16, GEMM_OUT_F32, GEMM_OUT_F32_ADD = 0, 1, 2
GEMM_A_K_MAJOR, GEMM_B_K_MAJOR = 1, 2


class Problem(ctypes.Structure):
    """struct vsce_problem."""
    _fields_ = [
        ("rows", c_int64),
        ("vocab", c_int64),
        ("row_stride", c_int64),
        ("dtype", c_int32),
        ("reduction", c_int32),
        ("target", c_void_p),
        ("class_weight", c_void_p),
        ("ignore_index", c_int64),
        ("label_smoothing", c_float),
        ("softcap", c_float),
        ("z_loss", c_float),
        ("flags", c_uint32),
        ("vocab_offset", c_int64),
        ("vocab_total", c_int64),
    ]


class FlceProblem(ctypes.Structure):
    """struct vsce_flce_problem."""
    _fields_ = [
        ("rows", c_int64),
        ("hidden", c_int64),
        ("vocab", c_int64),
        ("chunk_rows", c_int64),
        ("target", c_void_p),
        ("class_weight", c_void_p),
        ("ignore_index", c_int64),
        ("label_smoothing", c_float),
        ("softcap", c_float),
        ("z_loss", c_float),
        ("reduction", c_int32),
    ]


class Outputs(ctypes.Structure):
    """struct vsce_outputs."""
    _fields_ = [
        ("loss", c_void_p),
        ("row_loss", c_void_p),
        ("token_acc", c_void_p),
        ("acc_mean", c_void_p),
        ("z_loss", c_void_p),
    ]


class VsceError(RuntimeError):
    def __init__(self, fn: str, code: int, msg: str):
        super().__init__(f"{fn} failed: {msg} ({code})")
        self.code = code


_lib = None


def _bind_torch_runtime() -> None:
    """Loads PyTorch's HIP runtime before libvsce.so, and initialises it
    when a GPU is present.

    libvsce.so asks the dynamic loader for ``libamdhip64.so.7``; PyTorch's
    libraries ask for ``libamdhip64.so`` and ship their own copy, whose soname
    is also ``libamdhip64.so.7``.  Loaded after torch, the library's request is
    met by torch's copy (the loader matches it by soname), so one HIP runtime
    serves both.  Loaded before torch, the request pulls in the system ROCm
    runtime, torch's request for the unversioned name then loads its own copy
    as well, and the process holds two HIP runtimes and two HSA runtimes over
    the same device (tests/test_abi_cpu.py shows both orders on the host).
    So the binding always brings torch's runtime in first."""
    import torch
    if torch.cuda.is_available():
        torch.cuda.init()


def load() -> ctypes.CDLL:
    """Load libvsce.so from the package directory (build it with
    ``python -m vocab_softmax_cross_amd.build``), after PyTorch's HIP
    runtime."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run `python -m vocab_softmax_cross_amd.build`")
    _bind_torch_runtime()
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.POINTER
    lib.vsce_workspace_bytes.argtypes = [c_int64]
    lib.vsce_workspace_bytes.restype = c_size_t
    lib.ce_forward_fused_inplace.argtypes = [P(Problem), c_void_p, P(Outputs), c_void_p, c_void_p]
    lib.ce_forward_fused_inplace.restype = ctypes.c_int
    lib.ce_forward_fused_inplace_timed.argtypes = [P(Problem), c_void_p, P(Outputs), c_void_p,
                                                   c_void_p, c_void_p, c_void_p]
    lib.ce_forward_fused_inplace_timed.restype = ctypes.c_int
    lib.ce_forward_fused_inplace_noalloc.argtypes = [P(Problem), c_void_p, P(Outputs), c_void_p]
    lib.ce_forward_fused_inplace_noalloc.restype = ctypes.c_int
    lib.ce_forward_stats.argtypes = [P(Problem), c_void_p, c_void_p, P(Outputs), c_void_p, c_void_p]
    lib.ce_forward_stats.restype = ctypes.c_int
    lib.ce_forward_stats_partial.argtypes = [P(Problem), c_void_p, c_void_p, c_void_p]
    lib.ce_forward_stats_partial.restype = ctypes.c_int
    lib.ce_merge_stats.argtypes = [P(Problem), c_void_p, c_int32, c_void_p, P(Outputs), c_void_p,
                                   c_void_p]
    lib.ce_merge_stats.restype = ctypes.c_int
    lib.ce_backward_from_stats.argtypes = [P(Problem), c_void_p, c_void_p, c_void_p, c_void_p,
                                           c_int64, c_void_p, c_void_p]
    lib.ce_backward_from_stats.restype = ctypes.c_int
    lib.ce_scale_grad.argtypes = [c_void_p, c_int64, c_int64, c_int64, c_int32, c_void_p, c_int64,
                                  c_int32, c_void_p]
    lib.ce_scale_grad.restype = ctypes.c_int
    lib.vsce_gemm_bf16_nt.argtypes = [c_void_p, c_int64, c_void_p, c_int64, c_void_p, c_int64,
                                      c_int64, c_int64, c_int64, c_int32, c_void_p]
    lib.vsce_gemm_bf16_nt.restype = ctypes.c_int
    lib.vsce_gemm_bf16.argtypes = [c_void_p, c_int64, c_void_p, c_int64, c_void_p, c_int64,
                                   c_int64, c_int64, c_int64, c_uint32, c_int32, c_void_p]
    lib.vsce_gemm_bf16.restype = ctypes.c_int
    lib.vsce_flce_workspace_bytes.argtypes = [P(FlceProblem)]
    lib.vsce_flce_workspace_bytes.restype = c_size_t
    lib.flce_forward_backward.argtypes = [P(FlceProblem), c_void_p, c_void_p, P(Outputs),
                                          c_void_p, c_int64, c_void_p, c_void_p, c_void_p,
                                          c_void_p]
    lib.flce_forward_backward.restype = ctypes.c_int
    lib.vsce_strerror.argtypes = [ctypes.c_int]
    lib.vsce_strerror.restype = ctypes.c_char_p
    lib.vsce_version.argtypes = []
    lib.vsce_version.restype = ctypes.c_int
    _lib = lib
    return lib


def _check(fn: str, code: int) -> int:
    if code != OK:
        raise VsceError(fn, code, load().vsce_strerror(code).decode())
    return code


def vsce_workspace_bytes(rows: int) -> int:
    return int(load().vsce_workspace_bytes(rows))


def vsce_version() -> int:
    return int(load().vsce_version())


def ce_forward_fused_inplace(problem: Problem, logits_inout: int, outputs: Outputs,
                             workspace: int, stream: int) -> int:
    return _check("ce_forward_fused_inplace", load().ce_forward_fused_inplace(
        ctypes.byref(problem), logits_inout, ctypes.byref(outputs), workspace, stream))


def ce_forward_fused_inplace_timed(problem: Problem, logits_inout: int, outputs: Outputs,
                                   workspace: int, stream: int, begin: int, end: int) -> int:
    return _check("ce_forward_fused_inplace_timed", load().ce_forward_fused_inplace_timed(
        ctypes.byref(problem), logits_inout, ctypes.byref(outputs), workspace, stream, begin, end))


def ce_forward_fused_inplace_noalloc(problem: Problem, logits_inout: int, outputs: Outputs,
                                     stream: int) -> int:
    return _check("ce_forward_fused_inplace_noalloc", load().ce_forward_fused_inplace_noalloc(
        ctypes.byref(problem), logits_inout, ctypes.byref(outputs), stream))


def ce_forward_stats(problem: Problem, logits: int, stats: int, outputs: Outputs,
                     workspace: int, stream: int) -> int:
    return _check("ce_forward_stats", load().ce_forward_stats(
        ctypes.byref(problem), logits, stats, ctypes.byref(outputs), workspace, stream))


def ce_forward_stats_partial(problem: Problem, logits: int, partial: int, stream: int) -> int:
    return _check("ce_forward_stats_partial", load().ce_forward_stats_partial(
        ctypes.byref(problem), logits, partial, stream))


def ce_merge_stats(problem: Problem, partials: int, shards: int, stats: int, outputs: Outputs,
                   workspace: int, stream: int) -> int:
    return _check("ce_merge_stats", load().ce_merge_stats(
        ctypes.byref(problem), partials, shards, stats, ctypes.byref(outputs), workspace, stream))


def ce_backward_from_stats(problem: Problem, logits: int, grad: int, stats: int,
                           grad_output: int, grad_output_stride: int, workspace: int,
                           stream: int) -> int:
    return _check("ce_backward_from_stats", load().ce_backward_from_stats(
        ctypes.byref(problem), logits, grad, stats, grad_output, grad_output_stride, workspace,
        stream))


def ce_scale_grad(grad: int, rows: int, vocab: int, row_stride: int, dtype: int,
                  grad_output: int, grad_output_stride: int, skip_if_one: int,
                  stream: int) -> int:
    return _check("ce_scale_grad", load().ce_scale_grad(
        grad, rows, vocab, row_stride, dtype, grad_output, grad_output_stride, skip_if_one,
        stream))


def raw_call(name: str, *args) -> int:
    """Call an entry point and return its code without raising (tests of the
    argument checks)."""
    return int(getattr(load(), name)(*args))


def vsce_gemm_bf16_nt(A: int, lda: int, B: int, ldb: int, C: int, ldc: int, M: int, N: int, K: int,
                      out_mode: int, stream: int) -> int:
    return _check("vsce_gemm_bf16_nt", load().vsce_gemm_bf16_nt(A, lda, B, ldb, C, ldc, M, N, K,
                                                                 out_mode, stream))


def vsce_gemm_bf16(A: int, lda: int, B: int, ldb: int, C: int, ldc: int, M: int, N: int, K: int,
                   layout: int, out_mode: int, stream: int) -> int:
    return _check("vsce_gemm_bf16", load().vsce_gemm_bf16(A, lda, B, ldb, C, ldc, M, N, K, layout,
                                                          out_mode, stream))


def vsce_flce_workspace_bytes(problem: FlceProblem) -> int:
    return int(load().vsce_flce_workspace_bytes(ctypes.byref(problem)))


def flce_forward_backward(problem: FlceProblem, hidden: int, weight: int, outputs: Outputs,
                          grad_output, grad_output_stride: int, grad_hidden: int,
                          grad_weight: int, workspace: int, stream: int) -> int:
    return _check("flce_forward_backward", load().flce_forward_backward(
        ctypes.byref(problem), hidden, weight, ctypes.byref(outputs), grad_output,
        grad_output_stride, grad_hidden, grad_weight, workspace, stream))
