"""Comparators of GPU results against the oracle (test infrastructure).

Gradients: an element passes if it is within one unit in the last place of
the buffer type of the oracle's exact value rounded once to that type
(``strict``), or, where the gradient is a difference of nearly equal terms
(label smoothing, fp32 buffers), within the error of evaluating that
difference in fp32 (``floor``):
    |g - g64| <= 2^-24 (|xt_c - lse| + log2 V + 8 + C_c) k_c
                 (p_c |sigma A + Z| + sigma eta |w_c| + sigma (1 - eps) w_y [c == y])
with xt the (soft-capped) logits, k_c the cap's slope 1 - tanh^2(x_c / s)
(1 without a cap), Z = sigma_z 2 lambda lse the z-loss coefficient (0
without), and C_c = 0 without a cap, else
    C_c = |xt_c| + |mt| + 4 |x_c| / s        (mt = the capped row maximum):
 - |xt_c| + |mt|: every exponent takes the difference of two capped logits,
   each an fp32 value computed from x; its rounding alone is up to
   2^-24 |xt| (half an ulp), in any fp32 evaluation (stored logits, uncapped,
   are exact and need no such term);
 - 4 |x_c| / s: the conditioning of the slope 4 q / (1 + q)^2,
   q = exp(-2 |x_c| / s), where the cap saturates: an fp32 exponent argument
   carries a relative error of about 2^-23, so q (and the slope) carries one
   of about 2 |x_c| / s * 2^-23.
The strict fraction must be 1 for bf16/fp16 buffers without label smoothing;
the floored fraction must be 1 everywhere.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np

import oracle

# (significand bits, minimum normal exponent) per buffer type
FORMATS = {"f32": (24, -126), "bf16": (8, -126), "f16": (11, -14)}


def ulp(v: np.ndarray, dtype: str) -> np.ndarray:
    """Spacing of the buffer type at |v| (the subnormal spacing near 0)."""
    p, emin = FORMATS[dtype]
    a = np.abs(np.asarray(v, dtype=np.float64))
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    e = np.maximum(e, emin)
    return np.exp2(e - (p - 1))


@dataclass
class GradReport:
    n: int
    strict_fail: int
    floor_fail: int
    max_ulp: float

    @property
    def strict_frac(self) -> float:
        return 1.0 - self.strict_fail / max(self.n, 1)


def grad_report(g: np.ndarray, g64: np.ndarray, dtype: str, x: np.ndarray, target: np.ndarray,
                stats: np.ndarray, cls: np.ndarray, scale: np.ndarray, eps: float,
                weight=None, sum_w=None, softcap: float = 0.0, z_loss: float = 0.0,
                scale_z=None) -> GradReport:
    """g: GPU gradient (fp64 copy), g64: oracle exact scaled gradient, rows
    aligned; x: stored logits; stats: oracle (m, d', x_y, S) of the capped
    logits; scale / scale_z: per-row factors of the cross-entropy and z-loss
    parts."""
    g = np.asarray(g, dtype=np.float64)
    rn = oracle.round_to(g64, dtype)
    u = ulp(rn, dtype)
    diff = np.abs(g - rn)
    # NaN where the oracle has NaN is a match
    both_nan = np.isnan(g) & np.isnan(g64)
    strict = (diff <= u) | both_nan
    n, V = g.shape
    w = np.ones(V) if weight is None else np.asarray(weight, np.float64)
    sw = float(V) if sum_w is None else float(sum_w)
    eta = eps / V
    floor_ok = strict.copy()
    bad_rows = np.where(~strict.all(axis=1))[0]
    for r in bad_rows:
        if cls[r] != 0:
            continue
        m, dp = stats[r, 0], stats[r, 1]
        lse = m + math.log1p(dp)
        if softcap > 0:
            xt = softcap * np.tanh(x[r] / softcap)
            slope = 1.0 / np.cosh(x[r] / softcap) ** 2
            cap_terms = np.abs(xt) + abs(m) + 4 * np.abs(x[r]) / softcap
        else:
            xt, slope, cap_terms = x[r], 1.0, 0.0
        p = np.exp(xt - lse)
        y = int(target[r])
        wy = w[y]
        A = (1 - eps) * wy + eta * sw
        sz = 0.0 if scale_z is None else scale_z[r]
        Z = sz * 2.0 * z_loss * lse
        sg = abs(scale[r])
        mag = p * abs(scale[r] * A + Z) + sg * eta * np.abs(w)
        mag[y] += sg * (1 - eps) * wy
        tol = 2.0 ** -24 * (np.abs(xt - lse) + math.log2(V) + 8 + cap_terms) * mag * slope
        floor_ok[r] |= np.abs(g[r] - g64[r]) <= tol + u[r]
    with np.errstate(invalid="ignore"):
        units = np.where(u > 0, diff / u, 0.0)
    units = np.where(both_nan, 0.0, units)
    return GradReport(int(g.size), int((~strict).sum()), int((~floor_ok).sum()),
                      float(np.nanmax(units)) if units.size else 0.0)


# Relative error allowed in a capped logit the library reports (the maximum
# and target logit of the split statistics and shard records), in units of
# 2^-24: s tanh(x / s) evaluated in fp32 to a few units relative.
CAPPED_VALUE_UNITS = 8


def rel_err(a, b) -> np.ndarray:
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    with np.errstate(invalid="ignore", divide="ignore"):
        e = np.abs(a - b) / np.maximum(np.abs(b), 1e-30)
    return np.where(np.isnan(a) & np.isnan(b), 0.0, e)


def assert_loss_close(gpu, ref, rtol=1e-5, what="loss"):
    e = rel_err(gpu, ref)
    assert np.all(e <= rtol), f"{what}: max relative error {np.nanmax(e):.3e} > {rtol:g}"
