"""Seeded synthetic inputs for the five cross-entropy workloads.

Both the tests (for the HIP library and for the oracle) and ``bench.py`` draw
their inputs here, and nothing else is shared between the two sides.  This
module computes no loss, gradient or statistic of the method; it only draws
random numbers and, for the two workloads that prescribe a target probability,
places the target logit where a prescribed softmax value puts it (with SciPy's
logsumexp over the other classes).

Recipe (every stream is a NumPy PCG64 generator keyed by a SeedSequence):

* logits: rows are drawn in blocks of ``BLOCK`` rows, block b from
  ``SeedSequence([seed, 4, b])``, as float32 N(0, 1) scaled by sigma, then
  rounded to the buffer type (round-to-nearest-even, by torch's CPU cast);
  any row range can therefore be regenerated on its own;
* targets: uniform integers in [0, V) from ``SeedSequence([seed, 1])``;
* ignored rows: exactly ``round(f * BT)`` rows, the first of a permutation from
  ``SeedSequence([seed, 2])``, get ``ignore_index`` (-100);
* class weights: float32 uniform in [0.5, 1.5) from ``SeedSequence([seed, 3])``;
* confidence levels: row n targets softmax probability 0.9, 0.99 or 0.999 by
  n mod 3; the target logit is solved in fp64 from the other (already rounded)
  logits and rounded fp64 -> fp32 -> buffer type, so the achieved probability
  is close to, not exactly, the level (the buffer type cannot hold it);
* dominant rows: ``round(f * BT)`` rows chosen by a permutation from
  ``SeedSequence([seed, 5])`` get a target probability drawn uniform in
  [0.99, 0.999) from the same stream, placed the same way.

The shapes, value distributions and mixes are those of the workloads the pages
benchmark (BT = 8192 rows of V = 128256 bf16 logits is the headline one); the
pages use random logits only, so no dataset is stood in for.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass
from typing import Optional, Tuple

import numpy as np
import torch

BLOCK = 256
IGNORE_INDEX = -100
_THREADS = max(1, min(16, os.cpu_count() or 1))

TORCH_DTYPES = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}
ELEM_BYTES = {"f32": 4, "bf16": 2, "f16": 2}


@dataclass(frozen=True)
class Workload:
    name: str
    BT: int
    V: int
    dtype: str
    sigma: float
    ignore_frac: float = 0.0
    label_smoothing: float = 0.0
    reductions: Tuple[str, ...] = ("mean",)
    grad_outputs: Tuple[float, ...] = (1.0,)
    weighted: bool = False
    levels: Optional[Tuple[float, ...]] = None     # per-row target probability by n mod len
    dominant_frac: float = 0.0                      # rows with p(target) ~ U[0.99, 0.999)
    modes: Tuple[str, ...] = ("fused",)
    accuracy: bool = False
    seed: int = 1

    @property
    def torch_dtype(self):
        return TORCH_DTYPES[self.dtype]

    @property
    def elem_bytes(self) -> int:
        return ELEM_BYTES[self.dtype]


WORKLOADS = {
    "tiny": Workload("tiny", 64, 1000, "f32", 1.0, ignore_frac=0.10, seed=1),
    "confidence": Workload("confidence", 4096, 32000, "bf16", 1.0,
                           levels=(0.9, 0.99, 0.999), modes=("fused", "split"), seed=2),
    "llm_head": Workload("llm_head", 8192, 128256, "bf16", 2.0, ignore_frac=0.05,
                         label_smoothing=0.1, grad_outputs=(1.0, 0.37),
                         modes=("fused", "split"), seed=3),
    "weighted": Workload("weighted", 16384, 151936, "bf16", 1.5, ignore_frac=0.05,
                         label_smoothing=0.1, reductions=("sum", "none"),
                         grad_outputs=(0.5,), weighted=True, modes=("fused", "split"),
                         seed=4),
    "wide_fp32": Workload("wide_fp32", 8192, 256000, "f32", 3.0, label_smoothing=0.05,
                          reductions=("none",), dominant_frac=0.2, modes=("split",),
                          accuracy=True, seed=5),
}


def with_rows(wl: Workload, BT: int, V: Optional[int] = None) -> Workload:
    """The same recipe at another size (tests use reduced sizes of each workload)."""
    d = dict(wl.__dict__)
    d["BT"] = BT
    if V is not None:
        d["V"] = V
    return Workload(**d)


def _rng(*key: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(list(key))))


def targets(wl: Workload) -> np.ndarray:
    t = _rng(wl.seed, 1).integers(0, wl.V, size=wl.BT, dtype=np.int64)
    n_ign = int(round(wl.ignore_frac * wl.BT))
    if n_ign:
        rows = _rng(wl.seed, 2).permutation(wl.BT)[:n_ign]
        t[rows] = IGNORE_INDEX
    return t


def class_weights(wl: Workload) -> Optional[np.ndarray]:
    if not wl.weighted:
        return None
    return _rng(wl.seed, 3).uniform(0.5, 1.5, size=wl.V).astype(np.float32)


def target_probabilities(wl: Workload) -> np.ndarray:
    """Per-row prescribed softmax(target) (NaN where none is prescribed)."""
    p = np.full(wl.BT, np.nan)
    if wl.levels:
        lv = np.asarray(wl.levels, dtype=np.float64)
        p = lv[np.arange(wl.BT) % len(lv)]
    n_dom = int(round(wl.dominant_frac * wl.BT))
    if n_dom:
        g = _rng(wl.seed, 5)
        rows = g.permutation(wl.BT)[:n_dom]
        p[rows] = g.uniform(0.99, 0.999, size=n_dom)
    return p


def _raw_block(wl: Workload, b: int) -> torch.Tensor:
    r0 = b * BLOCK
    r1 = min(wl.BT, r0 + BLOCK)
    a = _rng(wl.seed, 4, b).standard_normal((r1 - r0, wl.V), dtype=np.float32)
    a *= np.float32(wl.sigma)
    return torch.from_numpy(a).to(wl.torch_dtype)


def _place_targets(wl: Workload, blk: torch.Tensor, r0: int, tgt: np.ndarray,
                   prob: np.ndarray) -> None:
    from scipy.special import logsumexp
    for i in range(blk.shape[0]):
        n = r0 + i
        p = prob[n]
        y = tgt[n]
        if np.isnan(p) or y < 0 or y >= wl.V:
            continue
        row = blk[i].to(torch.float64).numpy().copy()
        row[y] = -np.inf
        xy = np.log(p) - np.log1p(-p) + logsumexp(row)
        blk[i, y] = torch.tensor(np.float32(xy)).to(wl.torch_dtype)


def logits_rows(wl: Workload, r0: int, r1: int, tgt: Optional[np.ndarray] = None) -> torch.Tensor:
    """Rows [r0, r1) of the workload's logits as a CPU tensor of the buffer type."""
    if tgt is None:
        tgt = targets(wl)
    prob = target_probabilities(wl)
    out = torch.empty((max(0, r1 - r0), wl.V), dtype=wl.torch_dtype)
    if r1 <= r0:
        return out

    def fill(b):
        blk = _raw_block(wl, b)
        s0 = b * BLOCK
        if not np.all(np.isnan(prob[s0:s0 + blk.shape[0]])):
            _place_targets(wl, blk, s0, tgt, prob)
        lo, hi = max(r0, s0), min(r1, s0 + blk.shape[0])
        out[lo - r0:hi - r0] = blk[lo - s0:hi - s0]

    blocks = range(r0 // BLOCK, (r1 - 1) // BLOCK + 1)
    if len(blocks) == 1:
        fill(blocks[0])
    else:  # blocks are independent streams: draw them on several threads
        with ThreadPoolExecutor(min(len(blocks), _THREADS)) as ex:
            list(ex.map(fill, blocks))
    return out


def logits(wl: Workload, tgt: Optional[np.ndarray] = None) -> torch.Tensor:
    return logits_rows(wl, 0, wl.BT, tgt)


def logits_device(wl: Workload, device, tgt: Optional[np.ndarray] = None,
                  row_stride: Optional[int] = None) -> torch.Tensor:
    """The whole logits matrix on ``device``, generated block by block on the host.

    With ``row_stride`` > V the rows live in a wider buffer (the returned tensor
    is the [BT, V] view)."""
    if tgt is None:
        tgt = targets(wl)
    stride = row_stride or wl.V
    buf = torch.empty((wl.BT, stride), dtype=wl.torch_dtype, device=device)
    view = buf[:, :wl.V]
    step = BLOCK * 8
    for r0 in range(0, wl.BT, step):
        r1 = min(wl.BT, r0 + step)
        view[r0:r1].copy_(logits_rows(wl, r0, r1, tgt))
    return view


def as_f64(t: torch.Tensor) -> np.ndarray:
    """Exact fp64 copy of stored values (bf16, f16 and f32 upcast exactly)."""
    return t.detach().to("cpu").to(torch.float64).numpy()
