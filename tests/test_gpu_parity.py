"""Parity of the HIP path (through the C ABI) with the fp64 oracle, on the GPU.

Tolerances (from the method's stated targets):
* losses (per row and reduced): 1e-5 relative (fp32 accumulation);
* gradient: within 1 ulp of the oracle's value rounded once to the buffer
  type; where label smoothing or an fp32 buffer makes the element a
  difference of nearly equal terms, within the fp32 evaluation floor instead
  (tests/compare.py) -- the strict fraction must be 1 for bf16 without
  label smoothing;
* true-class gradient in the confident regime: <= 0.5% relative;
* split-mode statistics: m and x_y bit-equal, d' 1e-5 relative, S absolute
  64 u sum|w x|.
"""
import math
import sys

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from tests.compare import CAPPED_VALUE_UNITS, assert_loss_close, grad_report, rel_err

pytestmark = pytest.mark.gpu

vf = pytest.importorskip("vocab_softmax_cross_amd.functional")


def _note(msg):
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


def _dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def _go_tensor(go, reduction, rows, dev):
    if reduction == "none":
        return torch.full((rows,), go, dtype=torch.float32, device=dev)
    return torch.tensor(go, dtype=torch.float32, device=dev)


def run(wl, mode, reduction, go, accuracy=False, row_stride=None, check_rows=None,
        x_host=None, tgt=None, inplace_backward=False, softcap=0.0, z_loss=0.0,
        long_rows_ring=False):
    """Runs one forward + backward through the C ABI and returns GPU results
    (host copies) next to the oracle's."""
    dev = _dev()
    _note(f"{wl.name} BT={wl.BT} V={wl.V} {wl.dtype} mode={mode} red={reduction} go={go} "
          f"stride={row_stride} softcap={softcap} z_loss={z_loss} ring={long_rows_ring}")
    feat = dict(softcap=softcap, z_loss=z_loss)
    tgt = W.targets(wl) if tgt is None else tgt
    w = W.class_weights(wl)
    x_host = W.logits(wl, tgt) if x_host is None else x_host
    stride = row_stride or wl.V
    buf = torch.zeros((wl.BT, stride), dtype=wl.torch_dtype, device=dev)
    if stride > wl.V:
        buf[:, wl.V:] = 7.0  # padding columns must survive untouched
    x = buf[:, :wl.V]
    x.copy_(x_host.to(dev))
    t = torch.from_numpy(tgt).to(dev)
    wt = None if w is None else torch.from_numpy(w).to(dev)
    eps = wl.label_smoothing
    go_t = _go_tensor(go, reduction, wl.BT, dev)
    if mode == "fused":
        res = vf.forward_fused_inplace(x, t, wt, -100, eps, reduction, row_loss=True,
                                       accuracy=accuracy, return_z_loss=True,
                                       long_rows_ring=long_rows_ring, **feat)
        vf.scale_grad(x, go_t, reduction)
        g = x
        stats = None
    else:
        res = vf.forward_stats(x, t, wt, -100, eps, reduction, row_loss=True, accuracy=accuracy,
                               return_z_loss=True, **feat)
        g = vf.backward_from_stats(x, t, res["stats"], go_t, res["workspace"], wt, -100, eps,
                                   reduction, out=x if inplace_backward else None, **feat)
        stats = res["stats"].cpu().numpy().astype(np.float64)
    torch.cuda.synchronize()
    if stride > wl.V:
        assert torch.all(buf[:, wl.V:] == 7.0), "padding columns were written"
    out = {
        "loss": res["loss"].cpu().numpy().astype(np.float64),
        "row_loss": res["row_loss"].cpu().numpy().astype(np.float64),
        "z_loss": res["z_loss"].cpu().numpy().astype(np.float64),
        "stats": stats,
        "status": vf.status(res["workspace"]),
        "acc": None if not accuracy else res["token_acc"].cpu().numpy().astype(np.float64),
        "acc_mean": None if not accuracy else float(res["acc_mean"].cpu()),
    }
    rows = np.arange(wl.BT) if check_rows is None else np.asarray(check_rows)
    out["grad"] = g[torch.from_numpy(rows).to(dev)].float().cpu().numpy().astype(np.float64) \
        if len(rows) else np.zeros((0, wl.V))
    return out, x_host, tgt, w


def reference(wl, x_host, tgt, w, reduction, go, rows=None, softcap=0.0, z_loss=0.0):
    """Oracle over all rows (losses, stats) and the gradient of `rows`."""
    BT = wl.BT
    nz = oracle.normalizer(tgt, wl.V, w)
    feat = dict(softcap=softcap, z_loss=z_loss)
    loss_rows = np.empty(BT)
    z_rows = np.empty(BT)
    stats = np.empty((BT, 4))
    am = np.empty(BT, np.int64)
    cls = np.empty(BT, np.int32)
    chunk = max(1, (1 << 26) // wl.V)
    for r0 in range(0, BT, chunk):
        r1 = min(BT, r0 + chunk)
        r = oracle.rows(W.as_f64(x_host[r0:r1]), tgt[r0:r1], w, -100, wl.label_smoothing,
                        want_grad=False, **feat)
        loss_rows[r0:r1], z_rows[r0:r1] = r.loss, r.z
        stats[r0:r1], am[r0:r1], cls[r0:r1] = r.stats, r.argmax, r.cls
    rows = np.arange(BT) if rows is None else np.asarray(rows)
    scale = oracle.grad_scale(reduction, nz.W, go, BT)
    scale_z = oracle.grad_scale(reduction, float(nz.n_valid), go, BT)
    g64 = np.zeros((len(rows), wl.V))
    for i0 in range(0, len(rows), chunk):
        sel = rows[i0:i0 + chunk]
        r = oracle.rows(W.as_f64(x_host[torch.from_numpy(sel)]), tgt[sel], w, -100,
                        wl.label_smoothing, want_grad=True, scale=scale[sel],
                        scale_z=scale_z[sel], **feat)
        gg = r.grad
        gg[r.cls != 0] = 0.0
        g64[i0:i0 + len(sel)] = gg
    acc, acc_mean = oracle.token_accuracy(am, tgt, cls)
    return {
        "loss": oracle.reduce_loss(loss_rows, cls, nz.W, reduction, z_rows, nz.n_valid),
        "z_loss": oracle.reduce_loss(z_rows, cls, float(nz.n_valid), reduction),
        "row_loss": loss_rows, "stats": stats, "cls": cls, "norm": nz, "scale": scale,
        "scale_z": scale_z, "rows": rows, "grad": g64, "acc": acc, "acc_mean": acc_mean,
        "softcap": softcap, "z": z_loss,
    }


def check(wl, out, ref, x_host, tgt, w, strict_bf16=None):
    cap, lam = ref["softcap"], ref["z"]
    assert_loss_close(out["loss"], ref["loss"], 1e-5, "reduced loss")
    assert_loss_close(out["row_loss"], ref["row_loss"], 1e-5, "row loss")
    if lam > 0:
        assert_loss_close(out["z_loss"], ref["z_loss"], 1e-5, "z-loss")
    else:
        assert np.all((out["z_loss"] == 0) | np.isnan(np.asarray(ref["loss"]))), "z-loss without one"
    rows = ref["rows"]
    rep = grad_report(out["grad"], ref["grad"], wl.dtype, W.as_f64(x_host[torch.from_numpy(rows)]),
                      tgt[rows], ref["stats"][rows], ref["cls"][rows], ref["scale"][rows],
                      wl.label_smoothing, w, ref["norm"].sum_w, cap, lam, ref["scale_z"][rows])
    print(f"  grad: n={rep.n} strict_fail={rep.strict_fail} floor_fail={rep.floor_fail} "
          f"max_ulp={rep.max_ulp:.2f}", flush=True)
    assert rep.floor_fail == 0, rep
    if strict_bf16 or (strict_bf16 is None and wl.dtype != "f32" and wl.label_smoothing == 0):
        assert rep.strict_fail == 0, rep
    if out["stats"] is not None:
        valid = ref["cls"] == 0
        s, r = out["stats"][valid], ref["stats"][valid]
        if cap > 0:  # capped values: the fp32 cap is good to a few units of 2^-24, relative
            for k in (0, 2):
                assert np.all(np.abs(s[:, k] - r[:, k])
                              <= CAPPED_VALUE_UNITS * 2.0 ** -24 * np.abs(r[:, k])), k
        else:
            np.testing.assert_array_equal(s[:, 0], r[:, 0])
            np.testing.assert_array_equal(s[:, 2], r[:, 2])
        assert np.all(rel_err(s[:, 1], r[:, 1]) <= 1e-5), np.max(rel_err(s[:, 1], r[:, 1]))
        if wl.label_smoothing > 0:
            xa = np.abs(W.as_f64(x_host[torch.from_numpy(np.where(valid)[0])]))
            if cap > 0:
                xa = np.abs(cap * np.tanh(xa / cap))
            wa = np.ones(wl.V) if w is None else np.abs(w.astype(np.float64))
            # fp32 summation, plus each capped term's own relative error
            bound = (64 + (CAPPED_VALUE_UNITS if cap > 0 else 0)) * 2.0 ** -24 * (xa @ wa)
            assert np.all(np.abs(s[:, 3] - r[:, 3]) <= bound)
        else:
            assert np.all(s[:, 3] == 0.0)
    if out["acc"] is not None:
        np.testing.assert_array_equal(out["acc"], ref["acc"])
        assert out["acc_mean"] == pytest.approx(ref["acc_mean"], rel=1e-6)
    assert out["status"]["n_valid"] == ref["norm"].n_valid
    assert out["status"]["n_invalid"] == ref["norm"].n_invalid
    assert out["status"]["W"] == pytest.approx(ref["norm"].W, rel=1e-12)


# ---------------------------------------------------------------- the workloads

@pytest.mark.parametrize("mode", ["fused", "split"])
def test_tiny(mode):
    wl = W.WORKLOADS["tiny"]
    out, xh, tgt, w = run(wl, mode, "mean", 1.0, accuracy=True)
    check(wl, out, reference(wl, xh, tgt, w, "mean", 1.0), xh, tgt, w)


@pytest.mark.parametrize("mode", ["fused", "split"])
def test_confidence_regime(mode):
    """softmax(target) ~ 0.9 / 0.99 / 0.999 by row: dx_y within 0.5% of fp64."""
    wl = W.WORKLOADS["confidence"]
    rows = np.arange(0, wl.BT, 8)
    out, xh, tgt, w = run(wl, mode, "mean", 1.0, check_rows=rows)
    ref = reference(wl, xh, tgt, w, "mean", 1.0, rows)
    check(wl, out, ref, xh, tgt, w)
    gy = out["grad"][np.arange(len(rows)), tgt[rows]]
    ry = ref["grad"][np.arange(len(rows)), tgt[rows]]
    lvl = rows % 3
    for i in range(3):
        e = np.max(rel_err(gy[lvl == i], ry[lvl == i])) * 100
        print(f"  dx_y max rel err level {i}: {e:.3f}%", flush=True)
        assert e <= 0.5


@pytest.mark.parametrize("mode", ["fused", "split"])
@pytest.mark.parametrize("go", [1.0, 0.37])
def test_llm_head_rows(mode, go):
    """The headline row length (V = 128256, bf16, eps = 0.1, 5% ignored) on 96
    rows, every gradient element checked."""
    wl = W.with_rows(W.WORKLOADS["llm_head"], 96)
    out, xh, tgt, w = run(wl, mode, "mean", go)
    check(wl, out, reference(wl, xh, tgt, w, "mean", go), xh, tgt, w)


@pytest.mark.parametrize("mode", ["fused", "split"])
@pytest.mark.parametrize("reduction", ["sum", "none"])
def test_weighted_rows(mode, reduction):
    wl = W.with_rows(W.WORKLOADS["weighted"], 64)
    out, xh, tgt, w = run(wl, mode, reduction, 0.5)
    check(wl, out, reference(wl, xh, tgt, w, reduction, 0.5), xh, tgt, w)


@pytest.mark.parametrize("mode", ["split", "fused"])
def test_wide_fp32_rows(mode):
    """V = 256000 fp32 with dominant targets: the streaming kernels (the row
    does not fit on chip), accuracy included."""
    wl = W.with_rows(W.WORKLOADS["wide_fp32"], 40)
    out, xh, tgt, w = run(wl, mode, "none", 1.0, accuracy=True)
    check(wl, out, reference(wl, xh, tgt, w, "none", 1.0), xh, tgt, w)


# ---------------------------------------------------------------- full sizes, sampled

def _sample_rows(BT, k=24, seed=0):
    r = np.random.default_rng(seed).choice(BT, size=k, replace=False)
    return np.sort(np.concatenate([r, [0, BT - 1]]))


@pytest.mark.parametrize("mode,go", [("fused", 1.0), ("split", 0.37), ("fused", 0.37),
                                     ("split", 1.0)])
def test_llm_head_full_size(mode, go):
    """BT = 8192, V = 128256 bf16 in the launch configuration the benchmark
    times: every row loss, the reduced loss and the statistics checked, the
    gradient on sampled rows."""
    wl = W.WORKLOADS["llm_head"]
    rows = _sample_rows(wl.BT)
    out, xh, tgt, w = run(wl, mode, "mean", go, check_rows=rows)
    check(wl, out, reference(wl, xh, tgt, w, "mean", go, rows), xh, tgt, w)


@pytest.mark.parametrize("reduction", ["sum", "none"])
def test_weighted_full_size(reduction):
    wl = W.WORKLOADS["weighted"]
    rows = _sample_rows(wl.BT, 16, 1)
    out, xh, tgt, w = run(wl, "fused", reduction, 0.5, check_rows=rows)
    check(wl, out, reference(wl, xh, tgt, w, reduction, 0.5, rows), xh, tgt, w)


def test_wide_fp32_full_size():
    wl = W.WORKLOADS["wide_fp32"]
    rows = _sample_rows(wl.BT, 16, 2)
    out, xh, tgt, w = run(wl, "split", "none", 1.0, accuracy=True, check_rows=rows)
    check(wl, out, reference(wl, xh, tgt, w, "none", 1.0, rows), xh, tgt, w)


# ---------------------------------------------------------------- soft-capping and z-loss
# Named by Liger-Kernel PR #1268 (What changed, Correctness) without formulas;
# the oracle's plain definitions: capped logits s tanh(x / s) and lambda lse^2.

FEATURES = [(30.0, 0.0), (0.0, 1e-4), (30.0, 1e-4)]


@pytest.mark.parametrize("softcap,z_loss", FEATURES)
@pytest.mark.parametrize("mode,go", [("fused", 1.0), ("split", 0.37)])
def test_softcap_z_loss_llm_head_rows(softcap, z_loss, mode, go):
    """The headline recipe (bf16, V = 128256, smoothing, ignored rows) on the
    on-chip fused kernel and the split pair, every gradient element checked."""
    wl = W.with_rows(W.WORKLOADS["llm_head"], 64)
    kw = dict(softcap=softcap, z_loss=z_loss)
    out, xh, tgt, w = run(wl, mode, "mean", go, accuracy=True, **kw)
    check(wl, out, reference(wl, xh, tgt, w, "mean", go, **kw), xh, tgt, w)


@pytest.mark.parametrize("reduction,go", [("mean", 0.5), ("sum", 0.5), ("none", 0.5)])
@pytest.mark.parametrize("mode", ["fused", "split"])
def test_softcap_z_loss_weighted_rows(reduction, go, mode):
    """Class weights: the mean divides the cross-entropy by W and the z-loss by
    the valid rows, so the two gradient scales differ."""
    wl = W.with_rows(W.WORKLOADS["weighted"], 48)
    kw = dict(softcap=15.0, z_loss=1e-3)
    out, xh, tgt, w = run(wl, mode, reduction, go, **kw)
    check(wl, out, reference(wl, xh, tgt, w, reduction, go, **kw), xh, tgt, w)


@pytest.mark.parametrize("mode", ["fused", "split"])
def test_softcap_z_loss_wide_fp32_rows(mode):
    """fp32 rows too long to keep on chip: the fused mode takes the streaming
    kernel that reads the row twice."""
    wl = W.with_rows(W.WORKLOADS["wide_fp32"], 24)
    kw = dict(softcap=50.0, z_loss=1e-4)
    out, xh, tgt, w = run(wl, mode, "none", 1.0, accuracy=True, **kw)
    check(wl, out, reference(wl, xh, tgt, w, "none", 1.0, **kw), xh, tgt, w)


@pytest.mark.parametrize("mode", ["fused", "split"])
@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
def test_softcap_saturating_logits(mode, dtype):
    """Logits far beyond a small cap: many capped values tie at +-s, the
    slope underflows, and the accuracy still follows the stored logits."""
    wl = _small("tiny", 40, 3000, dtype=dtype, sigma=40.0, ignore_frac=0.1, label_smoothing=0.1)
    kw = dict(softcap=5.0, z_loss=0.05)
    out, xh, tgt, w = run(wl, mode, "mean", 1.0, accuracy=True, **kw)
    check(wl, out, reference(wl, xh, tgt, w, "mean", 1.0, **kw), xh, tgt, w)


@pytest.mark.parametrize("V", [7, 1001])
@pytest.mark.parametrize("mode", ["fused", "split"])
def test_softcap_z_loss_scalar_path(V, mode):
    """Row lengths that do not fill 16-byte vectors (per-element path)."""
    wl = _small("llm_head", 21, V, ignore_frac=0.1)
    kw = dict(softcap=20.0, z_loss=1e-2)
    out, xh, tgt, w = run(wl, mode, "sum", 0.37, **kw)
    check(wl, out, reference(wl, xh, tgt, w, "sum", 0.37, **kw), xh, tgt, w)


def test_softcap_z_loss_llm_head_full_size():
    """BT = 8192, V = 128256 bf16 with both features, fused: every row loss,
    the reduced loss and z-loss, sampled gradient rows."""
    wl = W.WORKLOADS["llm_head"]
    rows = _sample_rows(wl.BT, 12, 3)
    kw = dict(softcap=30.0, z_loss=1e-4)
    out, xh, tgt, w = run(wl, "fused", "mean", 1.0, check_rows=rows, **kw)
    check(wl, out, reference(wl, xh, tgt, w, "mean", 1.0, rows, **kw), xh, tgt, w)


@pytest.mark.parametrize("V,softcap,z_loss", [(128256, 30.0, 0.0), (128256, 3.0, 1e-4),
                                              (32000, 30.0, 1e-4), (32000, 3.0, 0.0)])
@pytest.mark.parametrize("mode", ["fused", "split"])
def test_softcap_strict_bf16_without_smoothing(V, softcap, z_loss, mode):
    """bf16 rows without label smoothing, soft-capped: every gradient element
    within 1 ulp of the exact value rounded once (the strict bar, no floor).
    A cap of 3 puts most logits (sigma 2) outside the polynomial's range, so
    both forms of the cap are exercised."""
    wl = _small("llm_head", 48, V, label_smoothing=0.0)
    kw = dict(softcap=softcap, z_loss=z_loss)
    out, xh, tgt, w = run(wl, mode, "mean", 1.0, accuracy=True, **kw)
    check(wl, out, reference(wl, xh, tgt, w, "mean", 1.0, **kw), xh, tgt, w, strict_bf16=True)


@pytest.mark.parametrize("softcap", [1.0, 7.0, 30.0, 1000.0])
def test_softcap_value_on_a_grid(softcap):
    """The capped logit s tanh(x / s) the library computes, read back through
    the split statistics (x[y] of each row is one grid point, 8192 points over
    |x| <= 12 s): within a few units of 2^-24 relative, on both sides of the
    polynomial's range."""
    dev = _dev()
    BT, V = 8192, 64
    xs = np.linspace(-12 * softcap, 12 * softcap, BT).astype(np.float32)
    x = torch.zeros((BT, V), dtype=torch.float32)
    x[:, 0] = torch.from_numpy(xs)
    t = torch.zeros(BT, dtype=torch.int64)
    res = vf.forward_stats(x.to(dev), t.to(dev), softcap=softcap, reduction="none")
    st = res["stats"].cpu().numpy().astype(np.float64)
    exact = softcap * np.tanh(xs.astype(np.float64) / softcap)
    units = np.abs(st[:, 2] - exact) / np.maximum(np.abs(exact), 1e-30) / 2.0 ** -24
    central = np.abs(xs) <= 0.35 * softcap
    print(f"  capped value: central max {units[central].max():.2f}, outside max "
          f"{units[~central].max():.2f} units of 2^-24", flush=True)
    assert units[central].max() <= 4 and units[~central].max() <= CAPPED_VALUE_UNITS


@pytest.mark.parametrize("variant", ["weights", "softcap_z_loss"])
def test_short_rows_weighted_or_capped(variant):
    """The 512-thread shape that serves rows of 2049-4096 vectors (bf16
    V = 32000) with class weights and with a soft-cap plus z-loss, and an fp32
    row of the same shape (V = 16000) with class weights."""
    kw = dict(softcap=30.0, z_loss=1e-4) if variant == "softcap_z_loss" else {}
    base = "weighted" if variant == "weights" else "llm_head"
    for dtype, V in (("bf16", 32000), ("f32", 16000)):
        if variant != "weights" and dtype == "f32":
            continue
        wl = _small(base, 40, V, dtype=dtype, ignore_frac=0.1, label_smoothing=0.1)
        red = "sum" if variant == "weights" else "mean"
        out, xh, tgt, w = run(wl, "fused", red, 0.5, accuracy=True, **kw)
        check(wl, out, reference(wl, xh, tgt, w, red, 0.5, **kw), xh, tgt, w)


# ---------------------------------------------------------------- vocab-parallel shards
# TransformerEngine PR #2325 (dist_process_group): each rank holds a slice of
# the vocabulary, the per-row record (max, sum, target logit, scaled_x_sum) is
# gathered and merged, and the review asks that the 4th value be summed too.
# On one GPU the shards are column slices of one buffer, their records stacked.

def run_sharded(wl, edges, reduction, go, softcap=0.0, z_loss=0.0, x_host=None, tgt=None):
    dev = _dev()
    _note(f"{wl.name} BT={wl.BT} V={wl.V} {wl.dtype} shards={len(edges) - 1} red={reduction} "
          f"go={go} softcap={softcap} z_loss={z_loss}")
    tgt = W.targets(wl) if tgt is None else tgt
    w = W.class_weights(wl)
    x_host = W.logits(wl, tgt) if x_host is None else x_host
    x = x_host.to(dev)
    t = torch.from_numpy(tgt).to(dev)
    wt = None if w is None else torch.from_numpy(w).to(dev)
    eps, V, P = wl.label_smoothing, wl.V, len(edges) - 1
    parts = torch.empty((P, wl.BT, 8), dtype=torch.float32, device=dev)
    for s_, (a, b) in enumerate(zip(edges[:-1], edges[1:])):
        vf.forward_stats_partial(x[:, a:b], t, a, V, wt, -100, eps, softcap, out=parts[s_])
    res = vf.merge_stats(parts, t, V, wt, -100, eps, reduction, softcap, z_loss, row_loss=True,
                         accuracy=True, return_z_loss=True, dtype=wl.torch_dtype)
    go_t = _go_tensor(go, reduction, wl.BT, dev)
    g = torch.empty_like(x)
    for a, b in zip(edges[:-1], edges[1:]):
        vf.backward_from_stats(x[:, a:b], t, res["stats"], go_t, res["workspace"], wt, -100, eps,
                               reduction, out=g[:, a:b], softcap=softcap, z_loss=z_loss,
                               vocab_offset=a, vocab_total=V)
    torch.cuda.synchronize()
    out = {
        "loss": res["loss"].cpu().numpy().astype(np.float64),
        "row_loss": res["row_loss"].cpu().numpy().astype(np.float64),
        "z_loss": res["z_loss"].cpu().numpy().astype(np.float64),
        "stats": res["stats"].cpu().numpy().astype(np.float64),
        "status": vf.status(res["workspace"]),
        "acc": res["token_acc"].cpu().numpy().astype(np.float64),
        "acc_mean": float(res["acc_mean"].cpu()),
        "grad": g.float().cpu().numpy().astype(np.float64),
        "parts": parts.cpu().numpy(),
    }
    return out, x_host, tgt, w


def check_parts(wl, out, x_host, tgt, w, edges, softcap):
    """Each shard's record against the oracle's record of the same shard."""
    xa = W.as_f64(x_host)
    for s_, (a, b) in enumerate(zip(edges[:-1], edges[1:])):
        ref = oracle.partials(xa[:, a:b], tgt, a, wl.V, w, -100, wl.label_smoothing, softcap)
        got = out["parts"][s_].astype(np.float64)
        valid = (tgt >= 0) & (tgt < wl.V)
        first = out["parts"][s_][:, 5].view(np.int32)
        np.testing.assert_array_equal(first[valid], ref[valid, 5].astype(np.int64))
        np.testing.assert_array_equal(got[valid, 4], ref[valid, 4])
        tol = CAPPED_VALUE_UNITS * 2.0 ** -24 * np.abs(ref[valid][:, [0, 2]]) if softcap else 0.0
        assert np.all(np.abs(got[valid][:, [0, 2]] - ref[valid][:, [0, 2]]) <= tol)
        assert np.all(rel_err(got[valid, 1], ref[valid, 1]) <= 1e-5)
        assert np.all(got[~valid] == 0)


# Shard edges: even halves, uneven quarters (all 16-byte aligned), and three
# shards of which two start or end off a 16-byte boundary (per-element path).
LLM_EDGES = {"halves": [0, 64128, 128256], "quarters": [0, 24000, 64000, 100008, 128256],
             "ragged": [0, 40001, 90000, 128256]}


@pytest.mark.parametrize("edges", list(LLM_EDGES))
@pytest.mark.parametrize("reduction,go", [("mean", 1.0), ("none", 0.37)])
def test_vocab_shards_llm_head_rows(edges, reduction, go):
    wl = W.with_rows(W.WORKLOADS["llm_head"], 48)
    e = LLM_EDGES[edges]
    out, xh, tgt, w = run_sharded(wl, e, reduction, go)
    check_parts(wl, out, xh, tgt, w, e, 0.0)
    check(wl, out, reference(wl, xh, tgt, w, reduction, go), xh, tgt, w)


@pytest.mark.parametrize("softcap,z_loss", [(0.0, 0.0), (15.0, 1e-3)])
def test_vocab_shards_weighted_rows(softcap, z_loss):
    """Class weights (all V given to every shard), smoothing, mean: W and the
    class-weight sum come from the merge's normalizers."""
    wl = W.with_rows(W.WORKLOADS["weighted"], 40)
    e = [0, 50000, 100000, 151936]
    kw = dict(softcap=softcap, z_loss=z_loss)
    out, xh, tgt, w = run_sharded(wl, e, "mean", 0.5, **kw)
    check_parts(wl, out, xh, tgt, w, e, softcap)
    check(wl, out, reference(wl, xh, tgt, w, "mean", 0.5, **kw), xh, tgt, w)


def test_vocab_shards_wide_fp32_rows():
    wl = W.with_rows(W.WORKLOADS["wide_fp32"], 16)
    e = [0, 64000, 128000, 192000, 256000]
    out, xh, tgt, w = run_sharded(wl, e, "sum", 1.0, softcap=50.0, z_loss=1e-4)
    check_parts(wl, out, xh, tgt, w, e, 50.0)
    check(wl, out, reference(wl, xh, tgt, w, "sum", 1.0, softcap=50.0, z_loss=1e-4), xh, tgt, w)


def test_vocab_shards_maximum_tied_across_shards():
    """Equal row maxima in two shards: the merge keeps the first shard's exact
    d' and counts the second copy, and the accuracy follows the first copy."""
    wl = _small("llm_head", 24, 4096, ignore_frac=0.0, label_smoothing=0.1)
    tgt = W.targets(wl)
    tgt[::2] = 100  # half the rows target the first copy of the maximum
    xh = W.logits(wl, tgt).clone()
    xh[:, 100] = 30.0
    xh[:, 3000] = 30.0
    e = [0, 2048, 4096]
    out, xh, tgt, w = run_sharded(wl, e, "mean", 1.0, x_host=xh, tgt=tgt)
    check_parts(wl, out, xh, tgt, w, e, 0.0)
    check(wl, out, reference(wl, xh, tgt, w, "mean", 1.0), xh, tgt, w)
    assert np.all(out["acc"][::2] == 1.0) and np.all(out["acc"][1::2] == 0.0)


# ---------------------------------------------------------------- edge cases

def _small(name, BT, V, **kw):
    base = W.WORKLOADS[name]
    d = dict(base.__dict__)
    d.update(BT=BT, V=V, **kw)
    return W.Workload(**d)


@pytest.mark.parametrize("V", [1, 2, 3, 7, 8, 9, 1001, 4097, 65541])
@pytest.mark.parametrize("mode", ["fused", "split"])
def test_ragged_vocab_bf16(V, mode):
    """Row lengths that do not fill 16-byte vectors take the scalar path."""
    wl = _small("llm_head", 37, V, ignore_frac=0.1, label_smoothing=0.0)
    out, xh, tgt, w = run(wl, mode, "mean", 1.0, accuracy=True)
    check(wl, out, reference(wl, xh, tgt, w, "mean", 1.0), xh, tgt, w)


@pytest.mark.parametrize("V", [8, 64, 2048, 16384, 32768, 65536, 128264, 130568, 131072, 163840,
                               262144])
def test_every_resident_shape(V):
    """One row length per on-chip shape boundary (V - 8: a ragged last
    slot), including the exact capacity of the shape with a partial LDS slot
    (130560) and the headline row length (128256)."""
    wl = _small("llm_head", 9, V - 8 if V > 8 else V)
    out, xh, tgt, w = run(wl, "fused", "mean", 1.0, accuracy=True)
    check(wl, out, reference(wl, xh, tgt, w, "mean", 1.0), xh, tgt, w)


# ---------------------------------------------------------------- one row per CU, many rows
# Rows of 16321-32768 vectors with class weights or a soft-cap (bf16 V up to
# 262144), and unweighted ones past the overflow shapes, take the shapes that
# hold one row per CU (1024 threads, 16 or 24 register slots and LDS).  These
# cases give every CU several rows in turn, with ignored rows first, last and
# in runs, and check every row loss and every gradient element.

def _targets_with_ignored_runs(wl):
    t = W.targets(wl)
    BT = wl.BT
    t[:3] = -100                     # the first rows
    t[BT - 4:] = -100                # the last rows
    t[BT // 3:BT // 3 + 70] = -100   # a run of 70
    t[BT // 2] = t[BT // 2 + 1]      # two rows with the same target
    return t


@pytest.mark.parametrize("case,reduction,go", [
    ("weighted_bf16", "sum", 0.5), ("weighted_bf16", "none", 0.5), ("weighted_f32", "none", 0.5),
    ("softcap_bf16", "mean", 1.0), ("weighted_softcap_bf16", "mean", 0.5),
    ("long_bf16", "mean", 1.0), ("long_weighted_bf16", "sum", 0.5),
    ("long_confident_bf16", "mean", 1.0), ("long_f16", "none", 0.37)])
def test_one_row_per_cu_shapes_many_rows(case, reduction, go):
    """Every row loss and every gradient element of 600-700 rows.  The rows of
    more than 20480 vectors without a soft-cap take the online statistics
    pass (long_*), here also in the confident regime (targets at softmax
    0.9 / 0.99 / 0.999, no smoothing: every element within 1 ulp)."""
    cases = {  # (workload, BT, V, dtype, features)
        "weighted_bf16": ("weighted", 640, 151936, "bf16", {}),
        "weighted_f32": ("weighted", 600, 70000, "f32", {}),
        "softcap_bf16": ("llm_head", 600, 140000, "bf16", dict(softcap=30.0, z_loss=1e-4)),
        "weighted_softcap_bf16": ("weighted", 600, 160000, "bf16",
                                  dict(softcap=15.0, z_loss=1e-3)),
        "long_bf16": ("llm_head", 700, 200000, "bf16", {}),
        "long_weighted_bf16": ("weighted", 600, 200000, "bf16", {}),
        "long_confident_bf16": ("confidence", 600, 200000, "bf16", {}),
        "long_f16": ("llm_head", 600, 250000, "f16", {}),
    }
    name, BT, V, dtype, kw = cases[case]
    wl = _small(name, BT, V, dtype=dtype)
    tgt = W.targets(wl) if name == "confidence" else _targets_with_ignored_runs(wl)
    out, xh, tgt, w = run(wl, "fused", reduction, go, accuracy=True, tgt=tgt, **kw)
    ref = reference(wl, xh, tgt, w, reduction, go, **kw)
    check(wl, out, ref, xh, tgt, w)
    if name == "confidence":
        rows = np.arange(wl.BT)
        gy = out["grad"][rows, tgt]
        ry = ref["grad"][rows, tgt]
        assert np.max(rel_err(gy, ry)) <= 0.005


def test_one_row_per_cu_nan_propagates():
    """A NaN logit reaches its row's loss and gradient only, on the online
    statistics pass (bf16 V = 200000) and the two-pass one (V = 151936)."""
    dev = _dev()
    for V in (200000, 151936):
        wl = _small("llm_head", 6, V)
        tgt = W.targets(wl)
        tgt[:] = np.arange(6) * 7 + 3
        xh = W.logits(wl, tgt)
        xh[2, V - 5] = float("nan")
        xh[4, 0] = float("nan")
        x = xh.to(dev)
        t = torch.from_numpy(tgt).to(dev)
        res = vf.forward_fused_inplace(x, t, reduction="none")
        torch.cuda.synchronize()
        loss = res["loss"].cpu()
        assert math.isnan(loss[2]) and math.isnan(loss[4]), V
        assert torch.isfinite(loss[[0, 1, 3, 5]]).all(), V
        assert torch.isnan(x[2]).all() and torch.isnan(x[4]).all(), V
        assert torch.isfinite(x[[0, 1, 3, 5]]).all(), V


# ---------------------------------------------------------------- rows longer than the chip
# Fused rows past the largest on-chip shape (32768 vectors), and rows off
# 16-byte vectors, are read twice: by default the statistics kernel and the
# gradient kernel in place; with VSCE_FLAG_LONG_ROWS_RING, rows on 16-byte
# vectors without class weights take the one-launch LDS ring instead (the
# others keep the default).

RING = pytest.mark.parametrize("ring", [False, True], ids=["pair", "ring"])


@RING
@pytest.mark.parametrize("V,dtype", [(262152, "bf16"), (300000, "bf16"), (262152, "f16"),
                                     (131080, "f32")])
@pytest.mark.parametrize("reduction,go", [("mean", 1.0), ("none", 0.37)])
def test_long_rows(V, dtype, reduction, go, ring):
    """Just past the largest on-chip shape (one vector in the last stage),
    and a longer row; ignored rows, smoothing, accuracy."""
    wl = _small("llm_head", 10, V, dtype=dtype, ignore_frac=0.2)
    out, xh, tgt, w = run(wl, "fused", reduction, go, accuracy=True, long_rows_ring=ring)
    check(wl, out, reference(wl, xh, tgt, w, reduction, go), xh, tgt, w)


@RING
def test_long_rows_softcap_z_loss(ring):
    wl = _small("llm_head", 8, 270000, ignore_frac=0.1)
    kw = dict(softcap=30.0, z_loss=1e-4)
    out, xh, tgt, w = run(wl, "fused", "mean", 1.0, accuracy=True, long_rows_ring=ring, **kw)
    check(wl, out, reference(wl, xh, tgt, w, "mean", 1.0, **kw), xh, tgt, w)


@RING
def test_long_rows_maximum_tied_everywhere(ring):
    """Rows whose maximum sits in many lanes' shares (every 97th column), one
    row constant (every element is the maximum), one with its target at the
    first copy: the shares of all owning lanes are re-read and summed."""
    wl = _small("llm_head", 4, 262152, ignore_frac=0.0, label_smoothing=0.0)
    tgt = W.targets(wl)
    xh = W.logits(wl, tgt).clone()
    xh[0, ::97] = 12.0
    xh[1, :] = 1.5
    xh[2, 5::97] = 12.0
    tgt[2] = 5
    out, xh, tgt, w = run(wl, "fused", "mean", 1.0, accuracy=True, x_host=xh, tgt=tgt,
                          long_rows_ring=ring)
    check(wl, out, reference(wl, xh, tgt, w, "mean", 1.0), xh, tgt, w)
    assert out["acc"][2] == 1.0  # the first copy of the maximum is the target


@RING
@pytest.mark.parametrize("wl_name,V", [("weighted", 262152), ("llm_head", 262153),
                                       ("llm_head", 65541)])
def test_long_rows_weighted_or_off_vectors(wl_name, V, ring):
    """Class weights, and rows off 16-byte vectors (long and short): the pair
    whether or not the ring is asked for."""
    wl = _small(wl_name, 6, V, ignore_frac=0.2)
    red = "sum" if wl.weighted else "mean"
    out, xh, tgt, w = run(wl, "fused", red, 0.5, long_rows_ring=ring)
    check(wl, out, reference(wl, xh, tgt, w, red, 0.5), xh, tgt, w)


def test_ring_flag_leaves_rows_that_fit_on_chip():
    wl = _small("llm_head", 12, 128256)
    out, xh, tgt, w = run(wl, "fused", "mean", 1.0, accuracy=True, long_rows_ring=True)
    check(wl, out, reference(wl, xh, tgt, w, "mean", 1.0), xh, tgt, w)


@pytest.mark.parametrize("dtype", ["f16", "f32"])
@pytest.mark.parametrize("mode", ["fused", "split"])
def test_other_dtypes(dtype, mode):
    wl = _small("llm_head", 33, 12000, dtype=dtype)
    out, xh, tgt, w = run(wl, mode, "sum", 0.37)
    check(wl, out, reference(wl, xh, tgt, w, "sum", 0.37), xh, tgt, w)


@pytest.mark.parametrize("mode", ["fused", "split"])
def test_row_stride_wider_than_vocab(mode):
    wl = _small("llm_head", 20, 5000)
    out, xh, tgt, w = run(wl, mode, "mean", 1.0, row_stride=5016)
    check(wl, out, reference(wl, xh, tgt, w, "mean", 1.0), xh, tgt, w)


@pytest.mark.parametrize("mode", ["fused", "split"])
def test_all_rows_ignored(mode):
    wl = _small("tiny", 16, 300)
    tgt = np.full(16, -100, np.int64)
    out, xh, _, w = run(wl, mode, "mean", 1.0, tgt=tgt)
    assert math.isnan(float(out["loss"]))
    assert np.all(out["grad"] == 0.0)
    assert np.all(out["row_loss"] == 0.0)


@pytest.mark.parametrize("mode", ["fused", "split"])
def test_empty_batch(mode):
    wl = _small("tiny", 0, 100)
    dev = _dev()
    x = torch.zeros((0, 100), device=dev)
    t = torch.zeros(0, dtype=torch.int64, device=dev)
    for red in ("mean", "sum", "none"):
        if mode == "fused":
            res = vf.forward_fused_inplace(x, t, reduction=red)
        else:
            res = vf.forward_stats(x, t, reduction=red)
        torch.cuda.synchronize()
        if red == "mean":
            assert math.isnan(float(res["loss"]))
        elif red == "sum":
            assert float(res["loss"]) == 0.0
        else:
            assert res["loss"].numel() == 0


@pytest.mark.parametrize("mode", ["fused", "split"])
def test_bad_targets_flagged(mode):
    wl = _small("tiny", 12, 257, ignore_frac=0.0)
    tgt = W.targets(wl)
    tgt[3] = 257
    tgt[7] = -5
    out, xh, _, w = run(wl, mode, "none", 1.0, tgt=tgt)
    assert out["status"]["status"] & 1
    assert math.isnan(out["row_loss"][3]) and math.isnan(out["row_loss"][7])
    assert np.all(out["grad"][[3, 7]] == 0.0)
    good = [i for i in range(12) if i not in (3, 7)]
    ref = reference(wl, xh, tgt, w, "none", 1.0)
    assert_loss_close(out["row_loss"][good], ref["row_loss"][good])


@pytest.mark.parametrize("mode", ["fused", "split"])
def test_ignore_index_inside_vocab(mode):
    dev = _dev()
    wl = _small("tiny", 10, 64)
    tgt = W.targets(wl)
    tgt[::3] = 5
    xh = W.logits(wl, tgt)
    x = xh.to(dev)
    t = torch.from_numpy(tgt).to(dev)
    if mode == "fused":
        res = vf.forward_fused_inplace(x, t, ignore_index=5, reduction="none", row_loss=True)
        g = x
    else:
        res = vf.forward_stats(x, t, ignore_index=5, reduction="none", row_loss=True)
        g = vf.backward_from_stats(x, t, res["stats"], torch.ones(10, device=dev),
                                   res["workspace"], ignore_index=5, reduction="none")
    torch.cuda.synchronize()
    r = oracle.cross_entropy(W.as_f64(xh), tgt, None, 5, 0.0, "none")
    assert_loss_close(res["loss"].cpu().numpy(), r.loss)
    assert torch.all(g[::3] == 0)


def test_nan_logit_propagates():
    dev = _dev()
    wl = _small("tiny", 4, 100)
    tgt = W.targets(wl)
    xh = W.logits(wl, tgt)
    xh[2, 17] = float("nan")
    for mode in ("fused", "split"):
        x = xh.to(dev)
        t = torch.from_numpy(tgt).to(dev)
        if mode == "fused":
            res = vf.forward_fused_inplace(x, t, reduction="none")
            g = x
        else:
            res = vf.forward_stats(x, t, reduction="none")
            g = vf.backward_from_stats(x, t, res["stats"], torch.ones(4, device=dev),
                                       res["workspace"], reduction="none")
        torch.cuda.synchronize()
        loss = res["loss"].cpu()
        assert math.isnan(loss[2]) and torch.isfinite(loss[[0, 1, 3]]).all()
        assert torch.isnan(g[2]).all() and torch.isfinite(g[[0, 1, 3]]).all()


def test_grad_output_one_skips_and_next_below_scales():
    dev = _dev()
    wl = _small("llm_head", 8, 4096)
    tgt = W.targets(wl)
    xh = W.logits(wl, tgt)
    x = xh.to(dev)
    t = torch.from_numpy(tgt).to(dev)
    vf.forward_fused_inplace(x, t)
    g0 = x.clone()
    vf.scale_grad(x, torch.tensor(1.0, device=dev))
    torch.cuda.synchronize()
    assert torch.equal(x, g0)
    below = float(np.nextafter(np.float32(1.0), np.float32(0.0)))
    vf.scale_grad(x, torch.tensor(below, device=dev))
    expect = (g0.float() * below).to(torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.equal(x, expect)


def test_deterministic_repeat():
    dev = _dev()
    wl = W.with_rows(W.WORKLOADS["llm_head"], 64)
    tgt = W.targets(wl)
    xh = W.logits(wl, tgt)
    outs = []
    for _ in range(2):
        x = xh.to(dev)
        res = vf.forward_fused_inplace(x, torch.from_numpy(tgt).to(dev), label_smoothing=0.1)
        torch.cuda.synchronize()
        outs.append((x.cpu(), res["loss"].cpu()))
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])


# ---------------------------------------------------------------- autograd and host syncs

def _no_sync_case(wl, mode, reduction, go):
    """Forward and backward through the autograd entry point under torch's
    sync debug mode "error", then the loss and gradient against the oracle."""
    dev = _dev()
    _note(f"no-sync {wl.name} BT={wl.BT} V={wl.V} mode={mode} red={reduction} go={go} "
          f"weighted={wl.weighted} eps={wl.label_smoothing}")
    tgt = W.targets(wl)
    xh = W.logits(wl, tgt)
    w = W.class_weights(wl)
    x = xh.to(dev).requires_grad_(True)
    t = torch.from_numpy(tgt).to(dev)
    wt = None if w is None else torch.from_numpy(w).to(dev)
    gout = _go_tensor(go, reduction, wl.BT, dev)
    torch.cuda.synchronize()
    torch.cuda.set_sync_debug_mode("error")
    try:
        from vocab_softmax_cross_amd import cross_entropy
        loss = cross_entropy(x, t, wt, -100, wl.label_smoothing, reduction, mode=mode)
        loss.backward(gout)
    finally:
        torch.cuda.set_sync_debug_mode("default")
    torch.cuda.synchronize()
    ref = oracle.cross_entropy(W.as_f64(xh), tgt, w, -100, wl.label_smoothing, reduction,
                               go if reduction != "none" else np.full(wl.BT, go), wl.dtype)
    assert_loss_close(loss.detach().cpu().numpy(), ref.loss)
    rep = grad_report(x.grad.float().cpu().numpy(), ref.grad, wl.dtype, W.as_f64(xh), tgt,
                      ref.stats, ref.cls, ref.scale, wl.label_smoothing, w, ref.norm.sum_w)
    assert rep.floor_fail == 0, rep


@pytest.mark.parametrize("mode", ["fused", "split"])
@pytest.mark.parametrize("reduction,go", [("mean", 1.0), ("sum", 0.37), ("none", 0.37)])
@pytest.mark.parametrize("variant", ["plain", "smoothing", "weights"])
def test_no_host_sync(mode, reduction, go, variant):
    """Forward and backward under torch's sync debug mode "error" (the
    pages' no-host-sync test, here for mean too)."""
    wl = _small("llm_head", 64, 8000, weighted=(variant == "weights"),
                label_smoothing=0.1 if variant != "plain" else 0.0)
    _no_sync_case(wl, mode, reduction, go)


@pytest.mark.parametrize("mode", ["fused", "split"])
@pytest.mark.parametrize("reduction,go", [("none", 0.5), ("sum", 0.5), ("mean", 0.37)])
def test_no_host_sync_weighted_workload(mode, reduction, go):
    """The same at the weighted workload's row length (V = 151936 bf16, class
    weights, smoothing 0.1, 5% ignored rows), with grad_output != 1: the
    weighted one-row-per-CU kernel, the split pair and the in-place scale
    (Liger-Kernel PR #1622, Testing Done: no host sync with class weights)."""
    _no_sync_case(W.with_rows(W.WORKLOADS["weighted"], 48), mode, reduction, go)


def test_fused_second_backward_raises():
    dev = _dev()
    x = torch.randn(4, 64, device=dev, dtype=torch.bfloat16, requires_grad=True)
    t = torch.randint(0, 64, (4,), device=dev)
    from vocab_softmax_cross_amd import cross_entropy
    loss = cross_entropy(x, t)
    loss.backward(retain_graph=True)
    with pytest.raises(RuntimeError):
        loss.backward()


def test_fused_peak_memory_is_one_logits_tensor():
    """Forward + backward allocate O(rows) beyond the logits (linkedin#1290:
    peak memory equals one logits tensor)."""
    dev = _dev()
    wl = W.with_rows(W.WORKLOADS["llm_head"], 1024)
    tgt = W.targets(wl)
    x = W.logits(wl, tgt).to(dev).requires_grad_(True)
    t = torch.from_numpy(tgt).to(dev)
    from vocab_softmax_cross_amd import cross_entropy
    torch.cuda.synchronize()
    torch.cuda.reset_peak_memory_stats()
    base = torch.cuda.memory_allocated()
    loss = cross_entropy(x, t, label_smoothing=0.1)
    loss.backward()
    torch.cuda.synchronize()
    extra = torch.cuda.max_memory_allocated() - base
    assert extra <= 64 * wl.BT + (1 << 20), extra


def test_graph_capture_replays_match_eager():
    """The fused step captured in a HIP graph: every replay (with eager work
    and synchronizations in between) equals the eager result."""
    dev = _dev()
    wl = W.with_rows(W.WORKLOADS["llm_head"], 128)
    tgt = W.targets(wl)
    xh = W.logits(wl, tgt)
    t = torch.from_numpy(tgt).to(dev)
    pristine = xh.to(dev)
    x = pristine.clone()
    eager = vf.forward_fused_inplace(x, t, label_smoothing=0.1)
    torch.cuda.synchronize()
    eager_g, eager_l = x.clone(), eager["loss"].clone()

    static_x = pristine.clone()
    ws = vf.workspace_for(wl.BT, dev)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        vf.forward_fused_inplace(static_x, t, label_smoothing=0.1, workspace=ws)  # warm-up
    torch.cuda.current_stream().wait_stream(s)
    static_x.copy_(pristine)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        res = vf.forward_fused_inplace(static_x, t, label_smoothing=0.1, workspace=ws)
    for _ in range(3):
        static_x.copy_(pristine)
        res["loss"].fill_(float("nan"))  # each replay must write its own reduced loss
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(static_x, eager_g)
        assert torch.equal(res["loss"], eager_l)
        _ = (pristine.float() * 2).sum()  # unrelated eager work between replays


@pytest.mark.parametrize("reduction", ["none", "sum"])
@pytest.mark.parametrize("mode", ["fused", "split"])
def test_graph_capture_weighted_step(mode, reduction):
    """A whole step of the weighted workload's rows (V = 151936 bf16, class
    weights, smoothing 0.1) captured in a HIP graph: the fused forward and the
    in-place grad_output scale at 0.5, or the statistics forward and the
    in-place backward.  Every replay, with eager work and synchronizations in
    between, equals the eager step bit for bit."""
    dev = _dev()
    wl = W.with_rows(W.WORKLOADS["weighted"], 64)
    tgt = W.targets(wl)
    w = W.class_weights(wl)
    xh = W.logits(wl, tgt)
    t = torch.from_numpy(tgt).to(dev)
    wt = torch.from_numpy(w).to(dev)
    eps = wl.label_smoothing
    go = _go_tensor(0.5, reduction, wl.BT, dev)
    pristine = xh.to(dev)

    def step(x, ws):
        if mode == "fused":
            res = vf.forward_fused_inplace(x, t, wt, -100, eps, reduction, row_loss=True,
                                           workspace=ws)
            vf.scale_grad(x, go, reduction)
        else:
            res = vf.forward_stats(x, t, wt, -100, eps, reduction, row_loss=True, workspace=ws)
            vf.backward_from_stats(x, t, res["stats"], go, ws, wt, -100, eps, reduction, out=x)
        return res

    x = pristine.clone()
    eager = step(x, vf.workspace_for(wl.BT, dev))
    torch.cuda.synchronize()
    eager_g, eager_l, eager_r = x.clone(), eager["loss"].clone(), eager["row_loss"].clone()
    ref = oracle.cross_entropy(W.as_f64(xh), tgt, w, -100, eps, reduction, 1.0, None,
                               want_grad=False)
    assert_loss_close(eager_l.cpu().numpy().astype(np.float64), ref.loss)

    static_x = pristine.clone()
    ws = vf.workspace_for(wl.BT, dev)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step(static_x, ws)  # warm-up
    torch.cuda.current_stream().wait_stream(s)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        res = step(static_x, ws)
    for _ in range(3):
        static_x.copy_(pristine)
        res["loss"].fill_(float("nan"))  # each replay must write its own outputs
        res["row_loss"].fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(static_x, eager_g)
        assert torch.equal(res["loss"], eager_l) and torch.equal(res["row_loss"], eager_r)
        _ = (pristine.float() * 2).sum()  # unrelated eager work between replays


# ---------------------------------------------------------------- rows with an overflow
# Uncapped, unweighted rows a little past the largest two-rows-per-CU shape
# (16320 vectors on chip) keep that shape and read the rest, the overflow,
# twice: 3 or 6 more vectors per thread (bf16 / f16 V <= 155136 / 179712,
# fp32 V <= 77568 / 89856).

ONCHIP_VECTORS = 16320


def _overflow_case(V, dtype, label_smoothing=0.1, base="llm_head"):
    """Rows engineered around the overflow: the target in it, a dominant
    target in it (confident row), maxima tied between the chip and the
    overflow and within the overflow, and an ignored row."""
    wl = _small(base, 12, V, dtype=dtype, ignore_frac=0.0, label_smoothing=label_smoothing)
    tgt = W.targets(wl)
    xh = W.logits(wl, tgt)
    vec = 4 if dtype == "f32" else 8
    ov0 = ONCHIP_VECTORS * vec  # first overflow column
    assert ov0 < V
    c1, c2, c3, c4 = 100, ov0 + 7, ov0 + 5, V - 3
    tgt[0] = V - 1
    tgt[1] = ov0
    tgt[2] = ov0 + 1234 % (V - ov0)
    xh[2, int(tgt[2])] = 24.0
    for r, y in ((3, c1), (4, c2)):
        xh[r, c1] = xh[r, c2] = 16.0
        tgt[r] = y
    xh[5, c3] = xh[5, c4] = 16.0
    tgt[5] = c4
    xh[6, c3] = 16.0
    tgt[6] = c3
    tgt[7] = -100
    return wl, xh, tgt


@pytest.mark.parametrize("V,dtype", [(131072, "bf16"), (155136, "bf16"), (155144, "bf16"),
                                     (179712, "bf16"), (151936, "f16"), (70000, "f32"),
                                     (89856, "f32")])
@pytest.mark.parametrize("reduction,go", [("mean", 1.0), ("none", 0.37)])
def test_overflow_rows(V, dtype, reduction, go):
    """Every overflow shape, at its capacity and just past the one before;
    targets, maxima and ties inside the overflow."""
    wl, xh, tgt = _overflow_case(V, dtype)
    out, xh, tgt, w = run(wl, "fused", reduction, go, accuracy=True, x_host=xh, tgt=tgt)
    check(wl, out, reference(wl, xh, tgt, w, reduction, go), xh, tgt, w)
    assert out["acc"][3] == 1.0 and out["acc"][4] == 0.0 and out["acc"][5] == 0.0
    assert out["acc"][6] == 1.0


@pytest.mark.parametrize("V", [131072, 151936, 179712])
@pytest.mark.parametrize("reduction,go", [("sum", 0.5), ("none", 0.5)])
def test_overflow_rows_weighted(V, reduction, go):
    """Class weights on the rows the overflow shapes serve unweighted (these
    take one row per CU): the weighted logit sum taken in the gradient pass,
    with the same engineered targets and maxima."""
    wl, xh, tgt = _overflow_case(V, "bf16", base="weighted")
    assert W.class_weights(wl) is not None
    out, xh, tgt, w = run(wl, "fused", reduction, go, accuracy=True, x_host=xh, tgt=tgt)
    check(wl, out, reference(wl, xh, tgt, w, reduction, go), xh, tgt, w)


def test_overflow_rows_confident_without_smoothing():
    """A dominant target in the overflow without smoothing: the strict 1-ulp
    bar for every gradient element, and the loss of the confident row."""
    wl, xh, tgt = _overflow_case(151936, "bf16", label_smoothing=0.0)
    out, xh, tgt, w = run(wl, "fused", "none", 1.0, accuracy=True, x_host=xh, tgt=tgt)
    check(wl, out, reference(wl, xh, tgt, w, "none", 1.0), xh, tgt, w, strict_bf16=True)


def test_overflow_nan_propagates():
    """A NaN logit in the overflow reaches its row's loss and gradient only."""
    dev = _dev()
    wl = _small("llm_head", 4, 131072)
    tgt = W.targets(wl)
    xh = W.logits(wl, tgt)
    xh[2, ONCHIP_VECTORS * 8 + 9] = float("nan")
    x = xh.to(dev)
    t = torch.from_numpy(tgt).to(dev)
    res = vf.forward_fused_inplace(x, t, reduction="none")
    torch.cuda.synchronize()
    loss = res["loss"].cpu()
    assert math.isnan(loss[2]) and torch.isfinite(loss[[0, 1, 3]]).all()
    assert torch.isnan(x[2]).all() and torch.isfinite(x[[0, 1, 3]]).all()


@pytest.mark.parametrize("V", [131072, 179712])
def test_overflow_rows_padded_stride(V):
    """The overflow of rows that live in wider buffers: the padding columns
    past V stay untouched (the overflow's accesses stop at the row's end)."""
    wl, xh, tgt = _overflow_case(V, "bf16")
    out, xh, tgt, w = run(wl, "fused", "mean", 1.0, accuracy=True, x_host=xh, tgt=tgt,
                          row_stride=V + 1024)
    check(wl, out, reference(wl, xh, tgt, w, "mean", 1.0), xh, tgt, w)
