"""fp64 CPU oracle for the fused softmax cross-entropy -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline``
leg may import this package.  It never imports the HIP library and the library
never imports it; the two share nothing but the seeded inputs of ``workloads``.

The per-row arithmetic lives in ``vsce_oracle.c`` (plain fp64 C, OpenMP over
rows); this module marshals numpy arrays into it and does the batch-level steps
in numpy fp64:

* the reduction of the per-row losses (none / sum / mean over the
  target-weight sum W) -- Liger-Kernel PR #1622 "perf(flce): drop host syncs
  that do not feed the computation", Summary, forward bullet;
* the gradient scale (1/W for mean, 1 for sum and none, times grad_output) --
  TransformerEngine PR #2325 "change fused cross entropy backward grad to fp32
  and reduce one read/write", sequence diagram ("Apply grad_output scaling");
* the token accuracy, argmax == target over valid rows divided by the count --
  PR #1622 Summary;
* the single rounding of the exact gradient to the buffer type -- Liger-Kernel
  PR #1268 "perf(ce): single-shot dx_y gradient correction", commit message of
  linkedin#1329.

Readings where the pages are silent: a mean over zero valid rows is NaN (0/0,
as PyTorch); an invalid target (neither ignore_index nor in [0, V)) gives that
row a NaN loss, which reaches any reduction, and a zero gradient.
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess
from dataclasses import dataclass, field
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "vsce_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

DTYPES = {"f32": 0, "bf16": 1, "f16": 2}
VALID, IGNORED, INVALID = 0, 1, 2
REDUCTIONS = ("none", "mean", "sum")


def build(force: bool = False) -> str:
    """Compile vsce_oracle.c into liboracle.so with gcc (IEEE fp64, OpenMP)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + f".tmp{os.getpid()}"
        subprocess.check_call(
            ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", "-Wall",
             _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def _load():
    global _lib
    if _lib is None:
        lib = ctypes.CDLL(build())
        p = ctypes.c_void_p
        i64 = ctypes.c_int64
        lib.oracle_round.argtypes = [p, p, i64, ctypes.c_int]
        lib.oracle_round.restype = None
        lib.oracle_round_one.argtypes = [ctypes.c_double, ctypes.c_int]
        lib.oracle_round_one.restype = ctypes.c_double
        lib.oracle_normalizer.argtypes = [i64, p, i64, p, i64, p, p, p, p]
        lib.oracle_normalizer.restype = None
        d = ctypes.c_double
        lib.oracle_rows.argtypes = [i64, i64, p, p, p, i64, d, d, d, p, p, p, p, p, p, p, p]
        lib.oracle_rows.restype = None
        lib.oracle_partials.argtypes = [i64, i64, i64, i64, p, p, p, i64, d, d, p]
        lib.oracle_partials.restype = None
        lib.oracle_merge.argtypes = [i64, i64, p, p, i64, i64, p, p]
        lib.oracle_merge.restype = None
        lib.oracle_max_threads.argtypes = []
        lib.oracle_max_threads.restype = ctypes.c_int
        lib.oracle_set_threads.argtypes = [ctypes.c_int]
        lib.oracle_set_threads.restype = None
        _lib = lib
    return _lib


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def max_threads() -> int:
    """Threads the oracle's OpenMP loops use (OMP_NUM_THREADS or all cores)."""
    return int(_load().oracle_max_threads())


def set_threads(n: int) -> None:
    """Use `n` threads in the oracle's parallel loops from now on."""
    _load().oracle_set_threads(int(n))


def round_to(values: np.ndarray, dtype: str) -> np.ndarray:
    """Round fp64 values to the buffer type (RNE), returned exactly as fp64."""
    src = np.ascontiguousarray(values, dtype=np.float64)
    out = np.empty_like(src)
    _load().oracle_round(_ptr(src), _ptr(out), src.size, DTYPES[dtype])
    return out


@dataclass
class Normalizer:
    n_valid: int
    W: float          # target-weight sum over valid rows (the count without weights)
    sum_w: float      # class-weight sum over all V classes (V without weights)
    n_invalid: int


def normalizer(target: np.ndarray, V: int, weight: Optional[np.ndarray] = None,
               ignore_index: int = -100) -> Normalizer:
    t = np.ascontiguousarray(target, dtype=np.int64)
    w = None if weight is None else np.ascontiguousarray(weight, dtype=np.float64)
    nv = ctypes.c_int64()
    W = ctypes.c_double()
    sw = ctypes.c_double()
    ni = ctypes.c_int64()
    _load().oracle_normalizer(t.size, _ptr(t), V, _ptr(w), ignore_index,
                              ctypes.byref(nv), ctypes.byref(W), ctypes.byref(sw),
                              ctypes.byref(ni))
    return Normalizer(nv.value, W.value, sw.value, ni.value)


@dataclass
class Rows:
    loss: np.ndarray       # [n] unreduced per-row loss (cross-entropy + z-loss)
    z: np.ndarray          # [n] the z-loss part alone
    stats: np.ndarray      # [n, 4] (m, d', x_y, S) of the (capped) logits
    argmax: np.ndarray     # [n] first index of the max of the stored logits
    cls: np.ndarray        # [n] 0 valid, 1 ignored, 2 invalid
    grad: Optional[np.ndarray]  # [n, V] dloss_n/dx with the per-row scales, or None


def rows(x: np.ndarray, target: np.ndarray, weight: Optional[np.ndarray] = None,
         ignore_index: int = -100, label_smoothing: float = 0.0,
         want_grad: bool = True, softcap: float = 0.0, z_loss: float = 0.0,
         scale: Optional[np.ndarray] = None, scale_z: Optional[np.ndarray] = None) -> Rows:
    """Per-row loss, statistics, argmax and gradient (see vsce_oracle.c).

    The gradient's cross-entropy part is multiplied by ``scale`` and its
    z-loss part by ``scale_z`` (per row; None: 1), before the softcap factor.
    """
    x = np.ascontiguousarray(x, dtype=np.float64)
    if x.ndim != 2:
        raise ValueError("x must be [rows, V]")
    n, V = x.shape
    t = np.ascontiguousarray(target, dtype=np.int64).reshape(n)
    w = None if weight is None else np.ascontiguousarray(weight, dtype=np.float64).reshape(V)
    sc = None if scale is None else np.ascontiguousarray(scale, dtype=np.float64).reshape(n)
    sz = None if scale_z is None else np.ascontiguousarray(scale_z, dtype=np.float64).reshape(n)
    loss = np.empty(n, np.float64)
    z = np.empty(n, np.float64)
    stats = np.empty((n, 4), np.float64)
    am = np.empty(n, np.int64)
    cls = np.empty(n, np.int32)
    grad = np.empty((n, V), np.float64) if want_grad else None
    _load().oracle_rows(n, V, _ptr(x), _ptr(t), _ptr(w), ignore_index,
                        float(label_smoothing), float(softcap), float(z_loss), _ptr(sc), _ptr(sz),
                        _ptr(loss), _ptr(z), _ptr(stats), _ptr(am), _ptr(cls), _ptr(grad))
    return Rows(loss, z, stats, am, cls, grad)


def partials(x_shard: np.ndarray, target: np.ndarray, v0: int, V: int,
             weight: Optional[np.ndarray] = None, ignore_index: int = -100,
             label_smoothing: float = 0.0, softcap: float = 0.0) -> np.ndarray:
    """One vocabulary shard's per-row record [n, 6]: (m_s, d'_s, x_y or 0,
    S_s, max of the stored logits, its first global column); see
    vsce_oracle.c."""
    x = np.ascontiguousarray(x_shard, dtype=np.float64)
    n, Vs = x.shape
    t = np.ascontiguousarray(target, dtype=np.int64).reshape(n)
    w = None if weight is None else np.ascontiguousarray(weight, dtype=np.float64).reshape(V)
    out = np.empty((n, 6), np.float64)
    _load().oracle_partials(n, Vs, v0, V, _ptr(x), _ptr(t), _ptr(w), ignore_index,
                            float(label_smoothing), float(softcap), _ptr(out))
    return out


def merge(parts: np.ndarray, target: np.ndarray, V: int, ignore_index: int = -100):
    """Shard records [P, n, 6] (column order) -> (stats [n, 4], argmax [n])."""
    pa = np.ascontiguousarray(parts, dtype=np.float64)
    P, n, _ = pa.shape
    t = np.ascontiguousarray(target, dtype=np.int64).reshape(n)
    stats = np.empty((n, 4), np.float64)
    am = np.empty(n, np.int64)
    _load().oracle_merge(n, P, _ptr(pa), _ptr(t), V, ignore_index, _ptr(stats), _ptr(am))
    return stats, am


def reduce_loss(row_loss: np.ndarray, cls: np.ndarray, W: float, reduction: str,
                row_z: Optional[np.ndarray] = None, n_valid: Optional[int] = None):
    """none -> the per-row vector; sum -> sum over rows; mean -> sum / W.

    With ``row_z`` (the z-loss part of each row loss), "mean" divides the
    cross-entropy part by W and the z-loss part by ``n_valid``: class weights
    weigh the cross-entropy only.  Ignored rows hold 0 and invalid rows NaN,
    so both enter the sums as they are.
    """
    if reduction == "none":
        return np.asarray(row_loss, dtype=np.float64).copy()

    def fsum(v):
        return math.fsum(float(e) for e in v) if not np.isnan(v).any() else math.nan

    if reduction == "sum":
        return fsum(row_loss)
    if reduction == "mean":
        if row_z is None:
            return fsum(row_loss) / W if W != 0 else math.nan
        ce = fsum(np.asarray(row_loss) - np.asarray(row_z))
        zs = fsum(row_z)
        return (ce / W if W != 0 else math.nan) + (zs / n_valid if n_valid else math.nan)
    raise ValueError(reduction)


def grad_scale(reduction: str, W: float, grad_output, n_rows: int) -> np.ndarray:
    """Per-row factor the unscaled gradient is multiplied by: grad_output times
    1/W (mean) or 1 (sum, none); grad_output is a scalar, or per row for none."""
    go = np.broadcast_to(np.asarray(grad_output, dtype=np.float64), (n_rows,)).copy() \
        if reduction == "none" else np.full(n_rows, float(np.asarray(grad_output).reshape(-1)[0]))
    if reduction == "mean":
        return go / W if W != 0 else np.full(n_rows, math.nan)
    return go


def token_accuracy(argmax: np.ndarray, target: np.ndarray, cls: np.ndarray):
    """Per-row 0/1 (valid and argmax == target) and its mean over valid rows."""
    valid = cls == VALID
    hit = (valid & (argmax == np.asarray(target))).astype(np.float64)
    nv = int(valid.sum())
    return hit, (float(hit.sum()) / nv if nv else math.nan)


@dataclass
class Result:
    loss: object                 # float (mean/sum) or [BT] array (none)
    z_loss: object               # the z-loss part, reduced like the loss
    row_loss: np.ndarray
    stats: np.ndarray
    argmax: np.ndarray
    cls: np.ndarray
    acc: np.ndarray
    acc_mean: float
    norm: Normalizer
    scale: np.ndarray            # [BT] per-row factor of the cross-entropy gradient
    scale_z: np.ndarray          # [BT] per-row factor of the z-loss gradient
    grad: Optional[np.ndarray] = None      # [BT, V] exact scaled gradient (fp64)
    grad_rn: Optional[np.ndarray] = None   # the same, rounded once to the buffer type
    extra: dict = field(default_factory=dict)


def cross_entropy(x: np.ndarray, target: np.ndarray, weight: Optional[np.ndarray] = None,
                  ignore_index: int = -100, label_smoothing: float = 0.0,
                  reduction: str = "mean", grad_output=1.0, dtype: Optional[str] = None,
                  want_grad: bool = True, softcap: float = 0.0, z_loss: float = 0.0) -> Result:
    """Whole-batch oracle for small inputs: everything the hot path computes.

    ``x`` holds the stored logits upcast exactly to fp64 ([BT, V]).  ``dtype``
    names the buffer type the gradient is rounded to (None: no rounding).
    """
    x = np.ascontiguousarray(x, dtype=np.float64)
    BT, V = x.shape
    nz = normalizer(target, V, weight, ignore_index)
    scale = grad_scale(reduction, nz.W, grad_output, BT)
    scale_z = grad_scale(reduction, float(nz.n_valid), grad_output, BT)
    r = rows(x, target, weight, ignore_index, label_smoothing, want_grad, softcap, z_loss,
             scale, scale_z)
    loss = reduce_loss(r.loss, r.cls, nz.W, reduction, r.z, nz.n_valid)
    zl = reduce_loss(r.z, r.cls, float(nz.n_valid), reduction)
    acc, acc_mean = token_accuracy(r.argmax, target, r.cls)
    res = Result(loss, zl, r.loss, r.stats, r.argmax, r.cls, acc, acc_mean, nz, scale, scale_z)
    if want_grad:
        res.grad = r.grad
        res.grad[r.cls != VALID] = 0.0
        if dtype is not None:
            res.grad_rn = round_to(res.grad, dtype)
    return res


# ---------------------------------------------------------------- FLCE
# The linear head fused with the cross-entropy (Liger-Kernel PR #1622
# "perf(flce): drop host syncs that do not feed the computation": the FLCE
# forward computes the loss and both gradients; the #1554 row compaction it
# mentions skips the projection products for ignored rows, which leaves every
# result unchanged).  Written as the definition:
#   z = h W^T                  (logits, [BT, V])
#   L = cross_entropy(z)       (the oracle above)
#   G = dL/dz                  (scaled by the reduction and grad_output)
#   dL/dh = G W,   dL/dW = G^T h
# in fp64 throughout, from the stored (bf16) h and W upcast exactly.

@dataclass
class FlceResult:
    ce: Result                 # the cross-entropy of z (loss, row losses, accuracy, G)
    logits: np.ndarray         # z = h W^T, fp64 [BT, V]
    grad_hidden: np.ndarray    # dL/dh, fp64 [BT, H]
    grad_weight: np.ndarray    # dL/dW, fp64 [V, H]


def matmul_nt(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """a b^T in fp64 ([M, K] x [N, K] -> [M, N]): the library product."""
    return np.asarray(a, np.float64) @ np.asarray(b, np.float64).T


def flce(hidden: np.ndarray, weight: np.ndarray, target: np.ndarray,
         class_weight: Optional[np.ndarray] = None, ignore_index: int = -100,
         label_smoothing: float = 0.0, reduction: str = "mean", grad_output=1.0,
         softcap: float = 0.0, z_loss: float = 0.0) -> FlceResult:
    """Loss and gradients of cross_entropy(hidden @ weight^T) in fp64."""
    h = np.asarray(hidden, np.float64)
    w = np.asarray(weight, np.float64)
    z = matmul_nt(h, w)
    ce = cross_entropy(z, target, class_weight, ignore_index, label_smoothing, reduction,
                       grad_output, None, True, softcap, z_loss)
    g = ce.grad
    return FlceResult(ce, z, g @ w, g.T @ h)
