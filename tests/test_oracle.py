"""Pins of the fp64 oracle against things other than itself (CPU only).

Each test ties one part of the oracle to a library routine, a closed form, an
invariant, 50-digit brute force, or the accuracy table printed on the pages,
so that a dropped term, a wrong sign or index, or a transposed operand in the
oracle fails at least one of them.
"""
import json
import math
import os

import mpmath
import numpy as np
import pytest
import torch
import torch.nn.functional as F
from scipy.special import logsumexp

import oracle
import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _problem(seed, BT, V, weighted=False, ignore_frac=0.0, sigma=1.0, dyadic=False):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((BT, V)) * sigma
    if dyadic:  # values that a bf16 buffer could hold, so shifts by 2^k stay exact
        x = np.round(x * 64) / 64
    t = rng.integers(0, V, BT).astype(np.int64)
    if ignore_frac:
        t[rng.permutation(BT)[: int(round(ignore_frac * BT))]] = -100
    w = rng.uniform(0.5, 1.5, V) if weighted else None
    return x, t, w


# ---------------------------------------------------------------- library routines

def test_unsmoothed_loss_is_logsumexp_minus_target_logit():
    x, t, _ = _problem(1, 32, 257, sigma=3.0)
    r = oracle.rows(x, t, want_grad=False)
    expect = logsumexp(x, axis=1) - x[np.arange(32), t]
    np.testing.assert_allclose(r.loss, expect, rtol=1e-13, atol=0)


@pytest.mark.parametrize("weighted", [False, True])
@pytest.mark.parametrize("eps", [0.0, 0.1, 0.7])
@pytest.mark.parametrize("reduction", ["none", "sum", "mean"])
def test_matches_torch_cross_entropy_fp64(weighted, eps, reduction):
    x, t, w = _problem(2, 24, 97, weighted=weighted, ignore_frac=0.25, sigma=2.0)
    go = np.linspace(0.3, 1.7, 24) if reduction == "none" else 0.37
    res = oracle.cross_entropy(x, t, w, -100, eps, reduction, go)

    xt = torch.tensor(x, dtype=torch.float64, requires_grad=True)
    wt = None if w is None else torch.tensor(w, dtype=torch.float64)
    lt = F.cross_entropy(xt, torch.tensor(t), weight=wt, ignore_index=-100,
                         reduction=reduction, label_smoothing=eps)
    lt.backward(torch.tensor(go, dtype=torch.float64) if reduction == "none"
                else torch.tensor(go, dtype=torch.float64))
    np.testing.assert_allclose(np.asarray(res.loss), lt.detach().numpy(), rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(res.grad, xt.grad.numpy(), rtol=1e-10, atol=1e-15)


def test_two_classes_is_the_logistic_loss():
    x, t, _ = _problem(3, 50, 2, sigma=4.0)
    r = oracle.rows(x, t, want_grad=False)
    other = x[np.arange(50), 1 - t]
    np.testing.assert_allclose(r.loss, np.logaddexp(0.0, other - x[np.arange(50), t]), rtol=1e-13)


def test_stats_and_argmax_match_numpy():
    x, t, w = _problem(4, 40, 301, weighted=True, sigma=2.0, dyadic=True)
    x[5, 17] = x[5, 200] = x[5].max() + 1.0        # a tie for the max: first index wins
    x[6, :] = 0.25                                  # every class ties
    r = oracle.rows(x, t, w, label_smoothing=0.2, want_grad=False)
    np.testing.assert_array_equal(r.argmax, np.argmax(x, axis=1))
    np.testing.assert_array_equal(r.stats[:, 0], x.max(axis=1))
    lse = logsumexp(x, axis=1)
    np.testing.assert_allclose(r.stats[:, 1], np.exp(lse - x.max(axis=1)) - 1.0, rtol=1e-12)
    np.testing.assert_array_equal(r.stats[:, 2], x[np.arange(40), t])
    np.testing.assert_allclose(r.stats[:, 3], x @ w, rtol=1e-12)
    r0 = oracle.rows(x, t, w, label_smoothing=0.0, want_grad=False)
    assert np.all(r0.stats[:, 3] == 0.0)


def test_token_accuracy_brute_force_with_ties():
    x, t, _ = _problem(5, 60, 11, ignore_frac=0.2, dyadic=True)
    x = np.floor(x * 2) / 2                         # coarse values: many ties
    t[:10] = np.argmax(x[:10], axis=1)              # some hits for sure
    res = oracle.cross_entropy(x, t, reduction="mean")
    hits, valid = 0, 0
    for n in range(60):
        if t[n] == -100:
            assert res.acc[n] == 0
            continue
        valid += 1
        best = 0
        for c in range(11):
            if x[n, c] > x[n, best]:
                best = c
        assert res.acc[n] == (1.0 if best == t[n] else 0.0)
        hits += best == t[n]
    assert res.acc_mean == hits / valid


# ---------------------------------------------------------------- brute force, 50 digits

def _mp_loss(xrow, y, w, eps):
    mpmath.mp.dps = 50
    V = len(xrow)
    w = [mpmath.mpf(1)] * V if w is None else [mpmath.mpf(float(v)) for v in w]

    def f(*xs):
        lse = mpmath.log(mpmath.fsum(mpmath.exp(v) for v in xs))
        s = mpmath.fsum(w[c] * (lse - xs[c]) for c in range(V))
        return (1 - mpmath.mpf(eps)) * w[y] * (lse - xs[y]) + mpmath.mpf(eps) / V * s
    return f


@pytest.mark.parametrize("V", [1, 2, 3, 5, 8])
@pytest.mark.parametrize("weighted,eps", [(False, 0.0), (False, 0.3), (True, 0.0), (True, 0.15)])
def test_brute_force_loss_and_derivative(V, weighted, eps):
    x, t, w = _problem(10 + V, 3, V, weighted=weighted, sigma=3.0)
    r = oracle.rows(x, t, w, label_smoothing=eps)
    for n in range(3):
        f = _mp_loss(x[n], int(t[n]), w, eps)
        pt = [mpmath.mpf(float(v)) for v in x[n]]
        assert float(r.loss[n]) == pytest.approx(float(f(*pt)), rel=1e-13, abs=1e-15)
        for c in range(V):
            d = [0] * V
            d[c] = 1
            g = mpmath.diff(f, pt, tuple(d))
            assert float(r.grad[n, c]) == pytest.approx(float(g), rel=1e-11, abs=1e-14)


def test_confident_rows_keep_d_prime_and_dxy_precision():
    """A dominant class: d' from 1e-2 down to 1e-9 must hold ~1e-12 relative,
    and so must dx_y = p_y - 1 (the cancellation the pages are about)."""
    mpmath.mp.dps = 50
    rng = np.random.default_rng(6)
    V = 64
    for gap in (5.0, 10.0, 15.0, 25.0):
        x = rng.standard_normal(V)
        y = 7
        x[y] = x.max() + gap
        r = oracle.rows(x[None, :], np.array([y]))
        mx = [mpmath.mpf(float(v)) for v in x]
        dp = mpmath.fsum(mpmath.exp(v - mx[y]) for i, v in enumerate(mx) if i != y)
        dxy = -dp / (1 + dp)
        assert float(r.stats[0, 1]) == pytest.approx(float(dp), rel=1e-12)
        assert float(r.grad[0, y]) == pytest.approx(float(dxy), rel=1e-12)
        assert float(r.loss[0]) == pytest.approx(float(mpmath.log1p(dp)), rel=1e-12)


# ---------------------------------------------------------------- finite differences of the reduced loss

@pytest.mark.parametrize("reduction", ["none", "sum", "mean"])
@pytest.mark.parametrize("weighted,eps", [(False, 0.0), (True, 0.2)])
def test_scaled_gradient_is_derivative_of_reduced_loss(reduction, weighted, eps):
    x, t, w = _problem(7, 5, 6, weighted=weighted, ignore_frac=0.2)
    go = np.array([0.5, 1.5, -0.7, 2.0, 0.3]) if reduction == "none" else 0.37
    res = oracle.cross_entropy(x, t, w, -100, eps, reduction, go)

    def J(xx):
        r = oracle.cross_entropy(xx, t, w, -100, eps, reduction, go, want_grad=False)
        return float(np.dot(go, r.loss)) if reduction == "none" else go * r.loss
    h = 1e-6
    fd = np.zeros_like(x)
    for n in range(5):
        for c in range(6):
            xp = x.copy()
            xm = x.copy()
            xp[n, c] += h
            xm[n, c] -= h
            fd[n, c] = (J(xp) - J(xm)) / (2 * h)
    np.testing.assert_allclose(res.grad, fd, rtol=1e-7, atol=1e-9)


# ---------------------------------------------------------------- closed forms and invariants

@pytest.mark.parametrize("weighted,eps", [(False, 0.0), (False, 0.1), (True, 0.0), (True, 0.3)])
def test_gradient_rows_sum_to_zero(weighted, eps):
    x, t, w = _problem(8, 16, 513, weighted=weighted, sigma=2.0)
    r = oracle.rows(x, t, w, label_smoothing=eps)
    s = r.grad.sum(axis=1)
    scale = np.abs(r.grad).sum(axis=1)
    assert np.all(np.abs(s) <= 1e-13 * scale)


@pytest.mark.parametrize("eps", [0.0, 0.1, 1.0])
def test_uniform_logits_closed_form(eps):
    V, BT = 1000, 8
    x = np.full((BT, V), 0.75)
    t = np.arange(BT) * 13
    res = oracle.cross_entropy(x, t, label_smoothing=eps, reduction="mean")
    assert res.loss == pytest.approx(math.log(V), rel=1e-14)
    expect = np.full((BT, V), 1.0 / V - eps / V)
    expect[np.arange(BT), t] -= 1.0 - eps
    np.testing.assert_allclose(res.grad, expect / BT, rtol=1e-12, atol=1e-18)


def test_one_class_has_zero_loss_and_gradient():
    x = np.array([[3.0], [-2.0], [0.0]])
    res = oracle.cross_entropy(x, np.zeros(3, np.int64), label_smoothing=0.1, reduction="none")
    assert np.all(res.loss == 0.0)
    assert np.all(res.grad == 0.0)


def test_shift_by_power_of_two_changes_nothing():
    x, t, w = _problem(9, 12, 129, weighted=True, dyadic=True)
    a = oracle.cross_entropy(x, t, w, label_smoothing=0.1, reduction="none")
    b = oracle.cross_entropy(x + 8.0, t, w, label_smoothing=0.1, reduction="none")
    np.testing.assert_allclose(a.loss, b.loss, rtol=1e-13)
    np.testing.assert_allclose(a.grad, b.grad, rtol=1e-12, atol=1e-17)


def test_uniform_class_weights():
    x, t, _ = _problem(10, 20, 50, ignore_frac=0.1)
    w = np.full(50, 2.5)
    plain_mean = oracle.cross_entropy(x, t, None, label_smoothing=0.1, reduction="mean")
    wmean = oracle.cross_entropy(x, t, w, label_smoothing=0.1, reduction="mean")
    plain_sum = oracle.cross_entropy(x, t, None, label_smoothing=0.1, reduction="sum")
    wsum = oracle.cross_entropy(x, t, w, label_smoothing=0.1, reduction="sum")
    assert wmean.loss == pytest.approx(plain_mean.loss, rel=1e-13)
    assert wsum.loss == pytest.approx(2.5 * plain_sum.loss, rel=1e-13)
    np.testing.assert_allclose(wmean.grad, plain_mean.grad, rtol=1e-12, atol=1e-18)


def test_ignored_rows_and_normalizer():
    x, t, w = _problem(11, 30, 40, weighted=True, ignore_frac=0.3)
    t[t == -100] = 5  # ignore_index inside [0, V) still ignores
    t[3] = 5
    res = oracle.cross_entropy(x, t, w, ignore_index=5, label_smoothing=0.1, reduction="mean")
    ign = t == 5
    assert np.all(res.row_loss[ign] == 0.0) and np.all(res.grad[ign] == 0.0)
    valid = (~ign)
    assert res.norm.n_valid == int(valid.sum())
    assert res.norm.W == pytest.approx(float(w[t[valid]].sum()), rel=1e-14)
    assert res.norm.sum_w == pytest.approx(float(w.sum()), rel=1e-14)
    assert res.loss == pytest.approx(float(res.row_loss.sum() / w[t[valid]].sum()), rel=1e-13)


def test_all_rows_ignored_mean_is_nan_with_zero_gradient():
    x, _, _ = _problem(12, 6, 10)
    t = np.full(6, -100)
    res = oracle.cross_entropy(x, t, reduction="mean")
    assert math.isnan(res.loss)
    assert np.all(res.grad == 0.0)
    xt = torch.tensor(x, requires_grad=True)
    assert math.isnan(float(F.cross_entropy(xt, torch.tensor(t), reduction="mean").detach()))


def test_invalid_target_gives_nan_loss_zero_gradient():
    x, t, _ = _problem(13, 5, 10)
    t[2] = 10
    t[4] = -3
    res = oracle.cross_entropy(x, t, reduction="none")
    assert math.isnan(res.row_loss[2]) and math.isnan(res.row_loss[4])
    assert np.all(res.grad[[2, 4]] == 0.0)
    assert res.norm.n_invalid == 2 and res.norm.n_valid == 3
    assert math.isnan(oracle.cross_entropy(x, t, reduction="sum").loss)


def test_nan_logit_reaches_loss_and_gradient():
    x, t, _ = _problem(14, 3, 10)
    x[1, 4] = np.nan
    res = oracle.cross_entropy(x, t, reduction="none")
    assert math.isnan(res.row_loss[1]) and np.all(np.isnan(res.grad[1]))
    assert np.all(np.isfinite(res.row_loss[[0, 2]]))


# ---------------------------------------------------------------- rounding to the buffer type

def _exact_rne(v, p, emin, emax):
    """Round-to-nearest-even with exact rational arithmetic (Python's round()
    on a Fraction rounds half to even)."""
    from fractions import Fraction
    if v == 0 or not math.isfinite(v):
        return v
    f = Fraction(v)
    e = math.floor(math.log2(abs(v)))
    while Fraction(2) ** e > abs(f):
        e -= 1
    while Fraction(2) ** (e + 1) <= abs(f):
        e += 1
    e = max(e, emin)
    q = Fraction(2) ** (e - p + 1)
    r = round(f / q) * q
    mx = (2 - Fraction(2) ** (1 - p)) * Fraction(2) ** emax
    if abs(r) > mx:
        return math.copysign(math.inf, v)
    return float(r)


def _rounding_cases(seed):
    rng = np.random.default_rng(seed)
    mags = np.exp2(rng.uniform(-140, 130, 4000))
    vals = mags * rng.choice([-1.0, 1.0], 4000) * (1 + rng.uniform(0, 1, 4000))
    # exact halfway points of bf16 and fp16 and values next to them
    base = rng.integers(1 << 7, 1 << 8, 200).astype(np.float64) * np.exp2(rng.integers(-20, 20, 200))
    half_bf16 = base + 0.5 * np.exp2(np.floor(np.log2(base)) - 7)
    half_f16 = base + 0.5 * np.exp2(np.floor(np.log2(base)) - 10)
    edge = np.array([65504.0, 65519.99, 65520.0, 3.3895313892515355e38, 3.3961775292304e38,
                     2.0 ** -133, 2.0 ** -134, 1.5 * 2.0 ** -134, 2.0 ** -24, 2.0 ** -25,
                     3.0 * 2.0 ** -26, 1e-45, 0.0, -0.0])
    return np.concatenate([vals, half_bf16, half_f16, np.nextafter(half_bf16, 0), edge])


def test_rounding_to_f32_matches_the_c_cast():
    v = _rounding_cases(20)
    with np.errstate(over="ignore"):
        np.testing.assert_array_equal(oracle.round_to(v, "f32"), v.astype(np.float32).astype(np.float64))


def test_rounding_to_f16_matches_numpy():
    v = _rounding_cases(21)
    with np.errstate(over="ignore"):
        np.testing.assert_array_equal(oracle.round_to(v, "f16"), v.astype(np.float16).astype(np.float64))


def test_rounding_to_bf16_matches_torch_and_exact_rationals():
    v = _rounding_cases(22)
    with np.errstate(over="ignore"):
        f32 = v.astype(np.float32)
    from_torch = torch.from_numpy(f32).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(oracle.round_to(f32.astype(np.float64), "bf16"), from_torch)
    exact = np.array([_exact_rne(float(a), 8, -126, 127) for a in v])
    np.testing.assert_array_equal(oracle.round_to(v, "bf16"), exact)


# ---------------------------------------------------------------- the pages' accuracy table

def test_reproduces_the_dxy_accuracy_table():
    """The table of maximum dx_y relative error (bf16, V=32000): an fp32
    evaluation rounded once stays under 0.5%, while the read-modify-write of
    the bf16 buffer reaches ~2%, ~20% and 100% at softmax(target) 0.9, 0.99,
    0.999.  Measured against the oracle's fp64 dx_y, on the confidence
    workload's recipe.  The row count is a power of two: the table's 1.95% at
    0.9 is exactly half a bf16 ulp of 0.9/N over 0.1/N (2^-9 / 0.1), which
    holds when N is a power of two; the pages do not state N."""
    with open(os.path.join(GOLDEN, "dxy_accuracy_table.json")) as fh:
        table = json.load(fh)
    wl = workloads.with_rows(workloads.WORKLOADS["confidence"], 2048)
    t = workloads.targets(wl)
    xb = workloads.logits(wl, t)
    x = workloads.as_f64(xb)
    N = wl.BT
    res = oracle.cross_entropy(x, t, reduction="mean", dtype="bf16")
    rows = np.arange(N)
    exact = res.grad[rows, t]

    # fp32 evaluation from the live max, sum and target logit, one rounding
    x32 = x.astype(np.float32)
    m = x32.max(axis=1)
    d = np.exp(x32 - m[:, None]).sum(axis=1, dtype=np.float32)
    py = np.exp(x32[rows, t] - m) / d
    fold = oracle.round_to((py - np.float32(1)) / np.float32(N), "bf16")
    # read-modify-write: softmax/N rounded into the bf16 buffer, then -1/N added
    stored = oracle.round_to((py / np.float32(N)).astype(np.float32), "bf16")
    rmw = oracle.round_to((stored.astype(np.float32) - np.float32(1.0 / N)).astype(np.float64), "bf16")

    level = np.arange(N) % 3
    for i, (p, before, at, _torch) in enumerate(table["rows"]):
        sel = level == i
        e_fold = np.max(np.abs(fold[sel] - exact[sel]) / np.abs(exact[sel])) * 100
        e_rmw = np.max(np.abs(rmw[sel] - exact[sel]) / np.abs(exact[sel])) * 100
        assert e_fold <= 0.5, (p, e_fold)
        assert e_fold == pytest.approx(before, abs=0.15), (p, e_fold, before)
        assert e_rmw == pytest.approx(at, rel=0.15), (p, e_rmw, at)


# ---------------------------------------------------------------- soft-capping and z-loss
# The pages name both features without a formula (Liger-Kernel PR #1268,
# What changed and Correctness); the oracle takes their plain definitions:
# capped logits s*tanh(x/s), and lambda * lse^2 per valid row.

def _torch_capped_ce(x, t, w, eps, reduction, softcap, z_loss, go=1.0):
    """Loss and input gradient through torch's own cross_entropy, tanh and
    autograd (fp64), with the z-loss mean taken over the valid rows."""
    xt = torch.tensor(x, dtype=torch.float64, requires_grad=True)
    capped = softcap * torch.tanh(xt / softcap) if softcap > 0 else xt
    tt = torch.tensor(t)
    wt = None if w is None else torch.tensor(w, dtype=torch.float64)
    valid = tt != -100
    ce = F.cross_entropy(capped, tt, weight=wt, ignore_index=-100, label_smoothing=eps,
                         reduction=reduction)
    z_rows = z_loss * torch.logsumexp(capped, dim=1) ** 2 * valid
    if reduction == "none":
        loss = ce + z_rows
        loss.backward(torch.as_tensor(go, dtype=torch.float64).expand_as(loss))
        return loss.detach().numpy(), xt.grad.numpy()
    z = z_rows.sum() / valid.sum() if reduction == "mean" else z_rows.sum()
    loss = ce + z
    (loss * go).backward()
    return float(loss.detach()), xt.grad.numpy()


@pytest.mark.parametrize("reduction", ["mean", "sum", "none"])
@pytest.mark.parametrize("weighted,eps", [(False, 0.0), (True, 0.1)])
@pytest.mark.parametrize("softcap,z_loss", [(30.0, 0.0), (0.0, 1e-3), (5.0, 0.2)])
def test_softcap_and_z_loss_match_torch_autograd(reduction, weighted, eps, softcap, z_loss):
    x, t, w = _problem(21, 24, 300, weighted=weighted, ignore_frac=0.2, sigma=6.0)
    go = np.linspace(0.5, 1.5, 24) if reduction == "none" else 0.7
    r = oracle.cross_entropy(x, t, w, label_smoothing=eps, reduction=reduction,
                             grad_output=go, softcap=softcap, z_loss=z_loss)
    ref_loss, ref_grad = _torch_capped_ce(x, t, w, eps, reduction, softcap, z_loss, go)
    np.testing.assert_allclose(r.loss, ref_loss, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(r.grad, ref_grad, rtol=1e-10, atol=1e-15)


def test_very_large_cap_is_plain_cross_entropy():
    x, t, w = _problem(22, 16, 200, weighted=True, sigma=2.0)
    a = oracle.cross_entropy(x, t, w, label_smoothing=0.1)
    b = oracle.cross_entropy(x, t, w, label_smoothing=0.1, softcap=1e7)
    assert b.loss == pytest.approx(a.loss, rel=1e-12)
    np.testing.assert_allclose(b.grad, a.grad, rtol=1e-9, atol=1e-16)


@pytest.mark.parametrize("z_loss", [0.0, 1e-4, 0.5])
def test_z_loss_uniform_logits_closed_form(z_loss):
    """Equal logits a: lse = a + log V, p = 1/V, loss = log V + lambda lse^2,
    dloss/dx_c = (1 + 2 lambda lse) / V - [c == y]."""
    V, a, y = 1000, 3.25, 17
    x = np.full((1, V), a)
    r = oracle.cross_entropy(x, np.array([y]), z_loss=z_loss, reduction="sum")
    lse = a + math.log(V)
    assert r.loss == pytest.approx(math.log(V) + z_loss * lse * lse, rel=1e-13)
    assert r.z_loss == pytest.approx(z_loss * lse * lse, rel=1e-13, abs=0)
    g = np.full(V, (1 + 2 * z_loss * lse) / V)
    g[y] -= 1.0
    np.testing.assert_allclose(r.grad[0], g, rtol=1e-12, atol=1e-16)
    assert r.stats[0, 0] == a and r.stats[0, 2] == a


def test_softcap_uniform_logits_closed_form():
    """Equal logits a capped at s: every capped logit is s tanh(a/s), so the
    loss is log V, and dloss/dx_c = (1/V - [c == y]) / cosh^2(a/s)."""
    V, a, y, s = 64, 7.0, 3, 5.0
    x = np.full((1, V), a)
    r = oracle.cross_entropy(x, np.array([y]), softcap=s, reduction="sum")
    assert r.loss == pytest.approx(math.log(V), rel=1e-13)
    g = np.full(V, 1.0 / V)
    g[y] -= 1.0
    np.testing.assert_allclose(r.grad[0], g / math.cosh(a / s) ** 2, rtol=1e-12)
    assert r.stats[0, 0] == pytest.approx(s * math.tanh(a / s), rel=1e-15)


def test_softcap_z_loss_gradient_is_finite_difference_of_loss():
    x, t, w = _problem(23, 3, 40, weighted=True, sigma=8.0)
    kw = dict(weight=w, label_smoothing=0.05, reduction="sum", softcap=6.0, z_loss=0.03)
    r = oracle.cross_entropy(x, t, **kw)
    h = 1e-4  # the loss is O(50): a smaller step drowns in fp64 roundoff
    for n in range(3):
        for c in (0, int(t[n]), 17, 39):
            xp, xm = x.copy(), x.copy()
            xp[n, c] += h
            xm[n, c] -= h
            fd = (oracle.cross_entropy(xp, t, **kw).loss
                  - oracle.cross_entropy(xm, t, **kw).loss) / (2 * h)
            assert r.grad[n, c] == pytest.approx(fd, rel=1e-6, abs=1e-9)


def test_softcap_z_loss_brute_force_50_digits():
    mpmath.mp.dps = 50
    x, t, w = _problem(24, 2, 12, weighted=True, sigma=9.0)
    s, lam, eps = 4.0, 0.07, 0.1
    r = oracle.rows(x, t, w, label_smoothing=eps, softcap=s, z_loss=lam)
    V = x.shape[1]
    wm = [mpmath.mpf(float(v)) for v in w]

    def loss_of(xs, y):
        xt = [mpmath.mpf(s) * mpmath.tanh(v / mpmath.mpf(s)) for v in xs]
        lse = mpmath.log(mpmath.fsum(mpmath.exp(v) for v in xt))
        sm = mpmath.fsum(wm[c] * (lse - xt[c]) for c in range(V))
        return ((1 - mpmath.mpf(eps)) * wm[y] * (lse - xt[y]) + mpmath.mpf(eps) / V * sm
                + mpmath.mpf(lam) * lse ** 2)

    for n in range(2):
        pt = [mpmath.mpf(float(v)) for v in x[n]]
        y = int(t[n])
        assert r.loss[n] == pytest.approx(float(loss_of(pt, y)), rel=1e-13)
        for c in (0, y, V - 1):
            d = [0] * V
            d[c] = 1
            g = mpmath.diff(lambda *v: loss_of(list(v), y), pt, tuple(d))
            assert r.grad[n, c] == pytest.approx(float(g), rel=1e-11, abs=1e-15)


def test_accuracy_uses_the_stored_logits_when_the_cap_saturates():
    """tanh(50) and tanh(60) are both 1.0 in fp64: the capped logits tie, but
    the prediction is the larger stored logit (capping is increasing)."""
    x = np.array([[500.0, 600.0, 0.0, -3.0]])
    r = oracle.cross_entropy(x, np.array([1]), softcap=10.0)
    assert r.argmax[0] == 1 and r.acc[0] == 1.0
    assert r.stats[0, 0] == 10.0                       # both capped to s
    assert r.stats[0, 1] == pytest.approx(1.0 + math.exp(-10.0) + math.exp(10 * math.tanh(-0.3) - 10))
    assert np.all(np.isfinite(r.grad))
    # the softcap factor 1/cosh^2 is below 1e-42 at 50 and 60
    assert abs(r.grad[0, 0]) < 1e-40 and abs(r.grad[0, 1]) < 1e-40


# ---------------------------------------------------------------- vocab-parallel merge
# TransformerEngine PR #2325: with a process group each rank holds a slice of
# the vocabulary and the per-row (max, sum, target logit, scaled_x_sum) record
# is gathered; its review comment asks that the 4th value be gathered and
# summed too.  The merge of the shards' records must give the unsharded row's
# statistics.

def _shard_edges(V, P, seed):
    if P == 1:
        return [0, V]
    rng = np.random.default_rng(seed)
    cuts = np.sort(rng.choice(np.arange(1, V), size=P - 1, replace=False))
    return [0, *cuts.tolist(), V]


def _merged(x, t, w, eps, softcap, edges):
    V = x.shape[1]
    parts = np.stack([oracle.partials(x[:, a:b], t, a, V, w, -100, eps, softcap)
                      for a, b in zip(edges[:-1], edges[1:])])
    return oracle.merge(parts, t, V)


@pytest.mark.parametrize("P", [1, 2, 3, 7])
@pytest.mark.parametrize("weighted,eps,softcap", [(False, 0.0, 0.0), (True, 0.1, 0.0),
                                                  (True, 0.1, 4.0)])
def test_merged_shard_statistics_equal_the_unsharded_row(P, weighted, eps, softcap):
    x, t, w = _problem(31, 20, 500, weighted=weighted, ignore_frac=0.2, sigma=3.0)
    r = oracle.rows(x, t, w, label_smoothing=eps, softcap=softcap, want_grad=False)
    stats, am = _merged(x, t, w, eps, softcap, _shard_edges(500, P, P))
    valid = r.cls == 0
    np.testing.assert_array_equal(stats[valid, 0], r.stats[valid, 0])   # the same element
    np.testing.assert_array_equal(stats[valid, 2], r.stats[valid, 2])   # the owner's value
    np.testing.assert_allclose(stats[valid, 1], r.stats[valid, 1], rtol=1e-13)
    np.testing.assert_allclose(stats[valid, 3], r.stats[valid, 3], rtol=1e-12, atol=1e-12)
    np.testing.assert_array_equal(am[valid], r.argmax[valid])
    assert np.all(stats[~valid] == 0)


def test_merge_with_the_maximum_tied_across_shards():
    """The row maximum sits in two shards: the merge excludes one copy and
    keeps the other (exp(0) = 1), and the argmax is the first occurrence."""
    x, t, _ = _problem(32, 6, 40, sigma=1.0)
    x[:, 7] = 5.0
    x[:, 30] = 5.0
    x[:, 31] = 5.0
    r = oracle.rows(x, t, want_grad=False)
    stats, am = _merged(x, t, None, 0.0, 0.0, [0, 10, 30, 40])
    np.testing.assert_allclose(stats[:, 1], r.stats[:, 1], rtol=1e-14)
    assert np.all(am == 7) and np.all(r.argmax == 7)
    assert np.all(stats[:, 1] >= 2.0)  # the two other copies count as exp(0) each


def test_dropping_the_summed_fourth_value_changes_it():
    """Negative control for the review comment: the smoothing sum S taken from
    one shard (not gathered and summed) differs from the row's S."""
    x, t, w = _problem(33, 8, 300, weighted=True, sigma=2.0)
    V = 300
    edges = [0, 100, 200, 300]
    parts = np.stack([oracle.partials(x[:, a:b], t, a, V, w, -100, 0.1)
                      for a, b in zip(edges[:-1], edges[1:])])
    r = oracle.rows(x, t, w, label_smoothing=0.1, want_grad=False)
    stats, _ = oracle.merge(parts, t, V)
    np.testing.assert_allclose(stats[:, 3], r.stats[:, 3], rtol=1e-12)
    assert np.all(np.abs(parts[0, :, 3] - r.stats[:, 3]) > 1e-3)


# ---------------------------------------------------------------- FLCE
# The linear head fused with the cross-entropy (Liger-Kernel PR #1622, the
# FLCE forward computing the loss and both gradients; #1554 compacts ignored
# rows out of the projection products without changing any result).

def _flce_problem(seed, BT, H, V, ignore_frac=0.25, weighted=False):
    rng = np.random.default_rng(seed)
    h = rng.standard_normal((BT, H))
    W = rng.standard_normal((V, H)) / math.sqrt(H) * 3.0
    t = rng.integers(0, V, BT).astype(np.int64)
    t[rng.permutation(BT)[: int(round(ignore_frac * BT))]] = -100
    cw = rng.uniform(0.5, 1.5, V) if weighted else None
    return h, W, t, cw


@pytest.mark.parametrize("reduction", ["mean", "sum", "none"])
@pytest.mark.parametrize("weighted,eps,softcap,z_loss", [(False, 0.0, 0.0, 0.0),
                                                         (True, 0.1, 0.0, 0.0),
                                                         (False, 0.1, 20.0, 1e-3)])
def test_flce_matches_torch_linear_cross_entropy_autograd(reduction, weighted, eps, softcap,
                                                          z_loss):
    h, W, t, cw = _flce_problem(41, 20, 24, 150, weighted=weighted)
    go = np.linspace(0.5, 1.5, 20) if reduction == "none" else 0.6
    r = oracle.flce(h, W, t, cw, -100, eps, reduction, go, softcap, z_loss)
    ht = torch.tensor(h, requires_grad=True)
    Wt = torch.tensor(W, requires_grad=True)
    z = F.linear(ht, Wt)
    zc = softcap * torch.tanh(z / softcap) if softcap > 0 else z
    tt = torch.tensor(t)
    valid = tt != -100
    ce = F.cross_entropy(zc, tt, weight=None if cw is None else torch.tensor(cw),
                         ignore_index=-100, label_smoothing=eps, reduction=reduction)
    zr = z_loss * torch.logsumexp(zc, dim=1) ** 2 * valid
    if reduction == "none":
        loss = ce + zr
        loss.backward(torch.tensor(go))
        np.testing.assert_allclose(r.ce.loss, loss.detach().numpy(), rtol=1e-12, atol=1e-14)
    else:
        loss = ce + (zr.sum() / valid.sum() if reduction == "mean" else zr.sum())
        (loss * go).backward()
        assert r.ce.loss == pytest.approx(float(loss), rel=1e-12)
    np.testing.assert_allclose(r.grad_hidden, ht.grad.numpy(), rtol=1e-10, atol=1e-14)
    np.testing.assert_allclose(r.grad_weight, Wt.grad.numpy(), rtol=1e-10, atol=1e-14)


def test_flce_gradients_are_finite_differences_of_the_loss():
    h, W, t, cw = _flce_problem(42, 6, 8, 40, weighted=True)
    kw = dict(class_weight=cw, label_smoothing=0.1, reduction="mean", softcap=10.0, z_loss=0.01)
    r = oracle.flce(h, W, t, **kw)
    d = 1e-5
    for (i, j) in [(0, 0), (2, 5), (5, 7)]:
        hp, hm = h.copy(), h.copy()
        hp[i, j] += d
        hm[i, j] -= d
        fd = (oracle.flce(hp, W, t, **kw).ce.loss - oracle.flce(hm, W, t, **kw).ce.loss) / (2 * d)
        assert fd == pytest.approx(r.grad_hidden[i, j], rel=1e-6, abs=1e-10)
    for (v, j) in [(0, 0), (int(t[t >= 0][0]), 3), (39, 7)]:
        Wp, Wm = W.copy(), W.copy()
        Wp[v, j] += d
        Wm[v, j] -= d
        fd = (oracle.flce(h, Wp, t, **kw).ce.loss - oracle.flce(h, Wm, t, **kw).ce.loss) / (2 * d)
        assert fd == pytest.approx(r.grad_weight[v, j], rel=1e-6, abs=1e-10)


def test_flce_ignored_rows_do_not_reach_the_gradients():
    """An ignored row's hidden state changes nothing: zero dL/dh row, the same
    loss and dL/dW (what makes skipping its products exact)."""
    h, W, t, _ = _flce_problem(43, 12, 16, 64, ignore_frac=0.5)
    r = oracle.flce(h, W, t, label_smoothing=0.1)
    ign = np.where(t == -100)[0]
    assert np.all(r.grad_hidden[ign] == 0.0)
    h2 = h.copy()
    h2[ign] = np.random.default_rng(0).standard_normal((len(ign), 16)) * 100
    r2 = oracle.flce(h2, W, t, label_smoothing=0.1)
    assert r2.ce.loss == r.ce.loss
    np.testing.assert_array_equal(r2.grad_weight, r.grad_weight)


@pytest.mark.parametrize("reduction", ["mean", "sum"])
def test_flce_on_the_compacted_rows_is_the_same(reduction):
    """Keeping only the valid rows (the compaction) gives the same loss, the
    same dL/dW and the valid rows' dL/dh."""
    h, W, t, cw = _flce_problem(44, 16, 8, 30, weighted=True)
    kw = dict(class_weight=cw, label_smoothing=0.05, reduction=reduction, grad_output=0.8)
    r = oracle.flce(h, W, t, **kw)
    keep = t != -100
    rc = oracle.flce(h[keep], W, t[keep], **kw)
    assert rc.ce.loss == pytest.approx(r.ce.loss, rel=1e-14)
    np.testing.assert_allclose(rc.grad_weight, r.grad_weight, rtol=1e-13, atol=1e-16)
    np.testing.assert_allclose(rc.grad_hidden, r.grad_hidden[keep], rtol=1e-13, atol=1e-16)
