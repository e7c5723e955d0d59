"""The linear head fused with the cross-entropy (FLCE) on the GPU, through the
C ABI, against the fp64 oracle.

The chain of checks:
* the bf16 GEMM against fp64 products, within the fp32-accumulation bound
  |c - c64| <= K 2^-24 sum_k |a b| (plus half a bf16 ulp when C is bf16);
* flce_forward_backward equals, bit for bit, the same stages composed from
  the public entry points (vsce_gemm_bf16_nt for z = h W^T, the fused
  cross-entropy on z, vsce_gemm_bf16_nt for G W and G^T h), with the ignored
  rows dropped on the host;
* each stage of that composition against the oracle on the stage's own
  inputs: the cross-entropy against oracle.cross_entropy of the bf16 logits
  (the cross-entropy tests' bars), the gradient products against fp64
  products of the bf16 G;
* end to end against oracle.flce (fp64, no intermediate rounding), within the
  first-order effect of rounding z to bf16, on small problems and at the
  benchmark's hidden size and vocabulary (H = 4096, V = 128256, 1000 rows);
* chunked runs against the unchunked one.
"""
import numpy as np
import pytest
import torch

import oracle
from tests.compare import assert_loss_close, grad_report

pytestmark = pytest.mark.gpu

vf = pytest.importorskip("vocab_softmax_cross_amd.functional")

U32 = 2.0 ** -24


def _dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def _note(msg):
    print(f"[case] {msg}", flush=True)


def _bf16(rng, shape, scale, dev):
    return torch.from_numpy((rng.standard_normal(shape) * scale).astype(np.float32)).to(
        torch.bfloat16).to(dev)


def _f64(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def _ulp_bf16(v):
    a = np.abs(v)
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    return np.exp2(np.maximum(e, -126) - 7)


def _check_product(got, a64, b64, bf16_out, what, add=None):
    exact = a64 @ b64.T + (0.0 if add is None else add)
    err = a64.shape[1] * U32 * (np.abs(a64) @ np.abs(b64).T)
    tol = err + (0.5 * _ulp_bf16(np.abs(exact) + err) if bf16_out else 0.0)
    bad = np.abs(got - exact) > tol
    assert not bad.any(), f"{what}: {bad.sum()} of {bad.size} outside the bound"


# ---------------------------------------------------------------- the GEMM

@pytest.mark.parametrize("M,N,K", [(128, 128, 64), (300, 260, 192), (64, 1000, 128),
                                   (1000, 4, 64), (257, 516, 4096)])
@pytest.mark.parametrize("mode", ["bf16", "f32", "f32_add"])
def test_gemm_matches_fp64(M, N, K, mode):
    dev = _dev()
    _note(f"gemm M={M} N={N} K={K} {mode}")
    rng = np.random.default_rng(M * 7 + N + K)
    a = _bf16(rng, (M, K), 1.0, dev)
    b = _bf16(rng, (N, K), 1.0, dev)
    if mode == "bf16":
        c = vf.gemm_bf16_nt(a, b)
        add = None
    else:
        c0 = torch.from_numpy(rng.standard_normal((M, N)).astype(np.float32)).to(dev)
        c = c0.clone()
        vf.gemm_bf16_nt(a, b, out=c, accumulate=(mode == "f32_add"))
        add = _f64(c0) if mode == "f32_add" else None
    torch.cuda.synchronize()
    _check_product(_f64(c), _f64(a), _f64(b), mode == "bf16", "gemm", add)


@pytest.mark.parametrize("M,N,K", [(1100, 16388, 128), (1100, 16392, 64), (200, 40000, 64)])
@pytest.mark.parametrize("mode", ["bf16", "f32_add"])
def test_gemm_workgroups_walk_several_tiles(M, N, K, mode):
    """More tiles than the chip holds workgroups (325 blocks of 256 x 256, 626
    of 128 x 128): each workgroup runs a sequence of tiles, loading the next
    tile's first stage while storing the last; K = 64 makes every step a
    tile's first and last.  N = 16388 takes the bf16 stores that stop at N
    (N not a multiple of 8), the others whole 16-byte chunks."""
    dev = _dev()
    _note(f"gemm M={M} N={N} K={K} {mode}")
    rng = np.random.default_rng(M + N + K)
    a = _bf16(rng, (M, K), 1.0, dev)
    b = _bf16(rng, (N, K), 1.0, dev)
    if mode == "bf16":
        c = vf.gemm_bf16_nt(a, b)
        add = None
    else:
        c0 = torch.from_numpy(rng.standard_normal((M, N)).astype(np.float32)).to(dev)
        c = c0.clone()
        vf.gemm_bf16_nt(a, b, out=c, accumulate=True)
        add = _f64(c0)
    torch.cuda.synchronize()
    _check_product(_f64(c), _f64(a), _f64(b), mode == "bf16", "gemm", add)


def _k_major(x, dev):
    """x [rows, K] as a transposed view of a [K, ld] buffer (ld a multiple of
    8 above rows), its padding columns NaN: only rows of C that are not
    stored may read them."""
    rows, K = x.shape
    ld = (rows + 8) // 8 * 8 + 8
    buf = torch.full((K, ld), float("nan"), dtype=torch.bfloat16, device=dev)
    buf[:, :rows] = x.t()
    return buf[:, :rows].t()


@pytest.mark.parametrize("layout", ["a", "b", "ab"])
@pytest.mark.parametrize("M,N,K", [(300, 260, 192), (1100, 16392, 64), (200, 4100, 128),
                                   (1100, 1004, 4096)])
@pytest.mark.parametrize("mode", ["bf16", "f32_add"])
def test_gemm_k_major_operands(layout, M, N, K, mode):
    """A and/or B read k-major in place ([K, rows] storage): within the fp64
    bound, and bit-identical to the row layout on the same values (the
    transposing LDS reads hand the MFMA the same operands, k in the same
    order)."""
    dev = _dev()
    _note(f"gemm k-major {layout} M={M} N={N} K={K} {mode}")
    rng = np.random.default_rng(M * 3 + N + K)
    a = _bf16(rng, (M, K), 1.0, dev)
    b = _bf16(rng, (N, K), 1.0, dev)
    ak = _k_major(a, dev) if "a" in layout else a
    bk = _k_major(b, dev) if "b" in layout else b
    assert (ak.stride(0) == 1) == ("a" in layout) and (bk.stride(0) == 1) == ("b" in layout)
    if mode == "bf16":
        c = vf.gemm_bf16_nt(ak, bk)
        ref = vf.gemm_bf16_nt(a, b)
        add = None
    else:
        c0 = torch.from_numpy(rng.standard_normal((M, N)).astype(np.float32)).to(dev)
        c, ref = c0.clone(), c0.clone()
        vf.gemm_bf16_nt(ak, bk, out=c, accumulate=True)
        vf.gemm_bf16_nt(a, b, out=ref, accumulate=True)
        add = _f64(c0)
    torch.cuda.synchronize()
    assert torch.equal(c.view(torch.int16) if mode == "bf16" else c.view(torch.int32),
                       ref.view(torch.int16) if mode == "bf16" else ref.view(torch.int32))
    _check_product(_f64(c), _f64(a), _f64(b), mode == "bf16", "k-major gemm", add)


def test_gemm_dh_at_the_full_vocabulary():
    """dL/dh = G W as the FLCE runs it at BT = 8192, H = 4096, V = 128256: W
    [V, H] read k-major in place, k running over the whole vocabulary (2004
    steps of 64), on 256 rows and 512 columns of the result against the fp64
    product.  G has the scale of a mean-reduced gradient."""
    dev = _dev()
    M, N, K = 256, 512, 128256
    _note(f"gemm dh M={M} N={N} K={K} (B k-major)")
    rng = np.random.default_rng(21)
    g = _bf16(rng, (M, K), 1.0 / 8192, dev)
    w = _bf16(rng, (K, N), 2.0 / np.sqrt(4096), dev)  # the head's weight, [V, H]
    c = vf.gemm_bf16_nt(g, w.t())
    torch.cuda.synchronize()
    _check_product(_f64(c), _f64(g), _f64(w).T, True, "dh = G W, K = 128256")


def test_gemm_dw_at_the_full_batch():
    """dL/dW = G^T h as the FLCE runs it at BT = 8192: G [BT, V] and h
    [BT, H] both read k-major in place, k running over the rows (128 steps of
    64), fp32 output, on 384 vocabulary rows and 512 hidden columns."""
    dev = _dev()
    M, N, K = 384, 512, 8192
    _note(f"gemm dW M={M} N={N} K={K} (A and B k-major)")
    rng = np.random.default_rng(22)
    g = _bf16(rng, (K, M), 1.0 / 8192, dev)  # G [BT, V] columns
    h = _bf16(rng, (K, N), 1.0, dev)         # h [BT, H]
    c = torch.empty((M, N), dtype=torch.float32, device=dev)
    vf.gemm_bf16_nt(g.t(), h.t(), out=c)
    torch.cuda.synchronize()
    _check_product(_f64(c), _f64(g).T, _f64(h).T, False, "dW = G^T h, K = 8192")


@pytest.mark.parametrize("dtype,N,ldc", [(torch.float32, 40, 48), (torch.bfloat16, 36, 44),
                                         (torch.bfloat16, 40, 48)])
def test_gemm_leaves_padding_alone(dtype, N, ldc):
    """Strided operands and output: columns past N of C are not written (bf16
    with N or ldc not a multiple of 8 stores 8 bytes at a time)."""
    dev = _dev()
    rng = np.random.default_rng(5)
    abuf = _bf16(rng, (96, 200), 1.0, dev)
    bbuf = _bf16(rng, (N, 200), 1.0, dev)
    a, b = abuf[:, :128], bbuf[:, :128]
    cbuf = torch.full((96, ldc), 7.0, dtype=dtype, device=dev)
    c = cbuf[:, :N]
    vf.gemm_bf16_nt(a, b, out=c)
    torch.cuda.synchronize()
    assert torch.all(cbuf[:, N:] == 7.0)
    _check_product(_f64(c), _f64(a), _f64(b), dtype == torch.bfloat16, "strided gemm")


# ---------------------------------------------------------------- FLCE

def _problem(seed, BT, H, V, ignore_frac=0.2, weighted=False):
    dev = _dev()
    rng = np.random.default_rng(seed)
    h = _bf16(rng, (BT, H), 1.0, dev)
    W = _bf16(rng, (V, H), 2.0 / np.sqrt(H), dev)
    t = rng.integers(0, V, BT).astype(np.int64)
    t[rng.permutation(BT)[: int(round(ignore_frac * BT))]] = -100
    cw = rng.uniform(0.5, 1.5, V).astype(np.float32) if weighted else None
    return h, W, t, cw


def _compose(h, W, t, cw, eps, reduction, softcap=0.0, z_loss=0.0):
    """The FLCE's stages through the public entry points, one chunk, the
    ignored rows dropped on the host: returns the stage inputs and outputs."""
    dev = h.device
    BT, H = h.shape
    V = W.shape[0]
    Vp = (V + 63) // 64 * 64
    keep = np.where(t != -100)[0]
    n = len(keep)
    C = (max(BT, 1) + 63) // 64 * 64
    xc = torch.zeros((C, H), dtype=torch.bfloat16, device=dev)
    xc[:n] = h[torch.from_numpy(keep).to(dev)]
    tc = np.full(C, -100, np.int64)
    tc[:n] = t[keep]
    Wp = torch.zeros((Vp, H), dtype=torch.bfloat16, device=dev)
    Wp[:V] = W
    z = torch.zeros((C, Vp), dtype=torch.bfloat16, device=dev)
    vf.gemm_bf16_nt(xc, Wp, out=z)
    z_bf = z.clone()
    zv = z[:, :V]
    cwt = None if cw is None else torch.from_numpy(cw).to(dev)
    res = vf.forward_fused_inplace(zv, torch.from_numpy(tc).to(dev), cwt, -100, eps, reduction,
                                   row_loss=True, softcap=softcap, z_loss=z_loss)
    G = z  # the gradient, in place, zero columns past V
    dxc = vf.gemm_bf16_nt(G, Wp.t().contiguous())
    dW = torch.empty((Vp, H), dtype=torch.float32, device=dev)
    vf.gemm_bf16_nt(G.t().contiguous(), xc.t().contiguous(), out=dW)
    torch.cuda.synchronize()
    return dict(keep=keep, n=n, tc=tc, z=z_bf, G=G, dxc=dxc, dW=dW[:V], res=res, xc=xc)


@pytest.mark.parametrize("reduction", ["mean", "sum"])
@pytest.mark.parametrize("weighted,eps", [(False, 0.0), (True, 0.1)])
def test_flce_equals_its_stages_and_each_stage_the_oracle(reduction, weighted, eps):
    h, W, t, cw = _problem(11, 300, 256, 1000, weighted=weighted)
    _note(f"flce BT=300 H=256 V=1000 red={reduction} weighted={weighted} eps={eps}")
    dev = h.device
    cwt = None if cw is None else torch.from_numpy(cw).to(dev)
    out = vf.flce_forward_backward(h, W, torch.from_numpy(t).to(dev), cwt, -100, eps, reduction,
                                   row_loss=True)
    st = _compose(h, W, t, cw, eps, reduction)
    torch.cuda.synchronize()
    keep, n = st["keep"], st["n"]
    # 1. The whole equals its stages, bit for bit.
    assert float(out["loss"]) == float(st["res"]["loss"])
    rl = np.zeros(300, np.float32)
    rl[keep] = st["res"]["row_loss"][:n].cpu().numpy()
    np.testing.assert_array_equal(out["row_loss"].cpu().numpy(), rl)
    gh = torch.zeros_like(h)
    gh[torch.from_numpy(keep).to(dev)] = st["dxc"][:n]
    assert torch.equal(out["grad_hidden"], gh)
    assert torch.equal(out["grad_weight"], st["dW"])
    # 2. The logits product against fp64.
    _check_product(_f64(st["z"][:n, :1000]), _f64(h)[keep], _f64(W), True, "z = h W^T")
    # 3. The cross-entropy stage against the oracle on the same bf16 logits.
    z64 = _f64(st["z"][:, :1000])
    ref = oracle.cross_entropy(z64, st["tc"], cw, -100, eps, reduction, 1.0, "bf16")
    assert_loss_close(float(st["res"]["loss"]), ref.loss, 1e-5, "chunk loss")
    g = _f64(st["G"][:, :1000])
    rep = grad_report(g, ref.grad, "bf16", z64, st["tc"], ref.stats, ref.cls, ref.scale, eps,
                      cw, ref.norm.sum_w)
    assert rep.floor_fail == 0, rep
    # 4. The gradient products against fp64 products of the bf16 G.
    g_n = g[:n]
    _check_product(_f64(st["dxc"][:n]), g_n, _f64(W).T, True, "dL/dh = G W")
    _check_product(_f64(st["dW"]), g_n.T, _f64(h)[keep].T, False, "dL/dW = G^T h")
    # 5. Ignored rows get zero dL/dh.
    assert torch.all(out["grad_hidden"][torch.from_numpy(np.where(t == -100)[0]).to(dev)] == 0)


@pytest.mark.parametrize("softcap,z_loss,reduction", [(0.0, 0.0, "mean"), (30.0, 1e-3, "sum"),
                                                       (15.0, 0.0, "none")])
def test_flce_end_to_end_against_the_fp64_oracle(softcap, z_loss, reduction):
    """The row losses within the first-order effect of rounding each logit to
    bf16 (|dl| <= sum_c |dl/dz_c| |dz_c| <= 2 max_c |dz_c|), the gradients
    within a bound of the same origin."""
    h, W, t, cw = _problem(12, 200, 512, 2048, weighted=True)
    _note(f"flce end to end softcap={softcap} z_loss={z_loss} red={reduction}")
    go = torch.linspace(0.5, 1.5, 200, device=h.device) if reduction == "none" else \
        torch.tensor(0.7, device=h.device)
    _end_to_end(h, W, t, cw, 0.05, reduction, softcap, z_loss, go)


def test_flce_at_the_full_hidden_size_and_vocabulary():
    """The FLCE at the hidden size and vocabulary of the pages' FLCE benchmark
    (H = 4096, V = 128256, bf16; Liger-Kernel PR #1622, host-blocking table),
    on 1000 rows (three full 256-row tiles and a ragged fourth, 5% ignored),
    smoothing 0.1, mean, through the same kernels bench.py times: every row
    loss and every element of dL/dh and dL/dW against the fp64 oracle, within
    the bounds of the small cases (z's product then runs K = 4096, dh's
    K = 128256)."""
    h, W, t, _ = _problem(31, 1000, 4096, 128256, ignore_frac=0.05)
    _note("flce end to end at H=4096 V=128256, 1000 rows")
    _end_to_end(h, W, t, None, 0.1, "mean", 0.0, 0.0, torch.tensor(1.0, device=h.device))


def _end_to_end(h, W, t, cw, eps, reduction, softcap, z_loss, go):
    dev = h.device
    BT, H = h.shape
    out = vf.flce_forward_backward(h, W, torch.from_numpy(t).to(dev),
                                   None if cw is None else torch.from_numpy(cw).to(dev), -100,
                                   eps, reduction, softcap, z_loss, grad_output=go,
                                   row_loss=True, accuracy=True, return_z_loss=True)
    torch.cuda.synchronize()
    h64, W64 = _f64(h), _f64(W)
    cw64 = None if cw is None else cw.astype(np.float64)
    go_host = go.cpu().numpy().astype(np.float64)
    ref = oracle.flce(h64, W64, t, cw64, -100, eps, reduction,
                      go_host if reduction == "none" else float(go_host), softcap, z_loss)
    z = ref.logits
    dz = 0.5 * _ulp_bf16(np.abs(z)) + H * U32 * (np.abs(h64) @ np.abs(W64).T)
    lse_term = 2.0 * z_loss * (np.abs(z).max(axis=1) + np.log(float(W.shape[0]))) + 2.0
    row_tol = lse_term * 1.5 * dz.max(axis=1) + 1e-5 * np.abs(ref.ce.row_loss)
    valid = t != -100
    got = out["row_loss"].cpu().numpy().astype(np.float64)
    assert np.all(np.abs(got - ref.ce.row_loss)[valid] <= row_tol[valid])
    assert np.all(got[~valid] == 0.0)
    # dL/dh and dL/dW, element by element, within the first-order effect of
    # the bf16 logits and the bf16 G (_grad_bounds).
    go_rows = go_host if reduction == "none" else np.full(BT, float(go_host))
    bh, bw = _grad_bounds(ref, h64, W64, dz, t, cw64, eps, softcap, z_loss, go_rows)
    gh = _f64(out["grad_hidden"])
    gw = out["grad_weight"].cpu().numpy().astype(np.float64)
    eh, ew = np.abs(gh - ref.grad_hidden), np.abs(gw - ref.grad_weight)
    print(f"  dL/dh: max error / bound {np.max(eh / bh):.3f}; dL/dW: {np.max(ew / bw):.3f}",
          flush=True)
    assert np.all(eh <= bh) and np.all(ew <= bw)
    assert np.all(gh[~valid] == 0.0)
    np.testing.assert_array_equal(out["token_acc"].cpu().numpy()[~valid], 0.0)


def _grad_bounds(ref, h64, W64, dz, t, cw, eps, softcap, z_loss, go_rows):
    """Element-wise bounds on dL/dh and dL/dW of the FLCE against the fp64
    oracle.  The library rounds each logit to bf16 (|dz_c| <= dz) and the
    cross-entropy gradient to bf16, then scales it in place by grad_output
    (a second rounding), before the two gradient products.  To first order,
    with xt the (capped) logits, k_c their slope, p = softmax(xt):
      |dp_c| <= p_c (k_c dz_c + max_j k_j dz_j)
      |dG_c| <= k_c |sigma A + Z| |dp_c| + (cap) |G_c / k_c| (2 |t_c| / s) dz_c
                + k_c p_c sigma_z 2 lambda max_j k_j dz_j
                + 1/2 go ulp_bf16(G_c / go) + 1/2 ulp_bf16(G_c)
    (Z = sigma_z 2 lambda lse, the z-loss coefficient; t_c = tanh(z_c / s);
    G and sigma include grad_output go), the first three terms with a 25%
    margin for second-order effects, then carried through the products with
    their own fp32 sums (and the bf16 rounding of dL/dh)."""
    BT, V = ref.logits.shape
    z = ref.logits
    G = ref.ce.grad
    w = np.ones(V) if cw is None else cw
    eta = eps / V
    sw = ref.ce.norm.sum_w
    dG = np.zeros_like(z)
    for n in range(BT):
        if t[n] == -100:
            continue
        m, dp = ref.ce.stats[n, 0], ref.ce.stats[n, 1]
        lse = m + np.log1p(dp)
        if softcap > 0:
            tt = np.tanh(z[n] / softcap)
            xt, k = softcap * tt, 1.0 - tt * tt
        else:
            xt, k, tt = z[n], np.ones(V), np.zeros(V)
        p = np.exp(xt - lse)
        sig, sz = ref.ce.scale[n], ref.ce.scale_z[n]
        A = (1 - eps) * w[t[n]] + eta * sw
        Z = sz * 2.0 * z_loss * lse
        kdz = k * dz[n]
        dmax = kdz.max()
        bound = k * abs(sig * A + Z) * p * (kdz + dmax) + k * p * abs(sz) * 2.0 * z_loss * dmax
        if softcap > 0:
            unsloped = abs(sig * A + Z) * p + abs(sig) * eta * w
            unsloped[t[n]] += abs(sig) * (1 - eps) * w[t[n]]
            bound += unsloped * (2.0 * np.abs(tt) / softcap) * dz[n]
        go = abs(go_rows[n])
        rounding = 0.5 * go * _ulp_bf16(np.abs(G[n]) / go) + 0.5 * _ulp_bf16(np.abs(G[n]))
        dG[n] = 1.25 * bound + rounding + 64 * U32 * np.abs(G[n])
    aG = np.abs(G)
    n_rows = BT
    bh = dG @ np.abs(W64) + V * U32 * (aG @ np.abs(W64))
    bh += 0.5 * _ulp_bf16(np.abs(ref.grad_hidden) + bh)
    bw = dG.T @ np.abs(h64) + n_rows * U32 * (aG.T @ np.abs(h64))
    return bh, bw


@pytest.mark.parametrize("chunk", [64, 128, 192])
def test_flce_chunked_equals_unchunked(chunk):
    """Chunks change nothing but the order of dL/dW's fp32 sums over rows."""
    h, W, t, cw = _problem(13, 500, 128, 640, weighted=False, ignore_frac=0.3)
    _note(f"flce chunk={chunk}")
    dev = h.device
    tt = torch.from_numpy(t).to(dev)
    a = vf.flce_forward_backward(h, W, tt, None, -100, 0.1, "mean", row_loss=True)
    b = vf.flce_forward_backward(h, W, tt, None, -100, 0.1, "mean", row_loss=True,
                                 chunk_rows=chunk)
    torch.cuda.synchronize()
    assert float(a["loss"]) == float(b["loss"])
    assert torch.equal(a["row_loss"], b["row_loss"])
    assert torch.equal(a["grad_hidden"], b["grad_hidden"])
    # dL/dW: two fp32 sums over the same n rows in different orders, each
    # within n 2^-24 sum_k |G||h| of the exact one (G from the stages, which
    # equal the unchunked run bit for bit).
    st = _compose(h, W, t, None, 0.1, "mean")
    n = st["n"]
    assert torch.equal(a["grad_weight"], st["dW"])
    g = np.abs(_f64(st["G"][:n, :640]))
    bound = 2 * n * U32 * (g.T @ np.abs(_f64(h)[st["keep"]]))
    diff = np.abs(_f64(a["grad_weight"]) - _f64(b["grad_weight"]))
    assert np.all(diff <= bound), float((diff - bound).max())


def test_flce_all_rows_ignored():
    h, W, t, _ = _problem(14, 70, 64, 128, ignore_frac=1.0)
    dev = h.device
    out = vf.flce_forward_backward(h, W, torch.from_numpy(t).to(dev), None, -100, 0.0, "sum")
    torch.cuda.synchronize()
    assert float(out["loss"]) == 0.0
    assert torch.all(out["grad_hidden"] == 0) and torch.all(out["grad_weight"] == 0)


@pytest.mark.parametrize("chunk", [0, 64])
def test_flce_rows_off_vectors_weighted_capped_per_row_grad_output(chunk):
    """V = 999 is not a multiple of 8, so the chunk's cross-entropy takes the
    statistics + gradient pair instead of the on-chip kernel; with class
    weights, soft-cap, z-loss and a grad_output per row (reduction none)."""
    h, W, t, cw = _problem(15, 150, 128, 999, weighted=True, ignore_frac=0.25)
    _note(f"flce V=999 chunk={chunk}")
    dev = h.device
    go = torch.linspace(0.25, 2.0, 150, device=dev)
    kw = dict(softcap=25.0, z_loss=1e-3)
    out = vf.flce_forward_backward(h, W, torch.from_numpy(t).to(dev),
                                   torch.from_numpy(cw).to(dev), -100, 0.1, "none",
                                   chunk_rows=chunk, grad_output=go, row_loss=True,
                                   return_z_loss=True, **kw)
    torch.cuda.synchronize()
    h64, W64 = _f64(h), _f64(W)
    ref = oracle.flce(h64, W64, t, cw.astype(np.float64), -100, 0.1, "none",
                      go.cpu().numpy().astype(np.float64), 25.0, 1e-3)
    valid = t != -100
    z = ref.logits
    dz = 0.5 * _ulp_bf16(np.abs(z)) + 128 * U32 * (np.abs(h64) @ np.abs(W64).T)
    tol = (3.0 + 2e-3 * (np.abs(z).max(axis=1) + np.log(999.0))) * dz.max(axis=1) \
        + 1e-5 * np.abs(ref.ce.row_loss)
    got = out["loss"].cpu().numpy().astype(np.float64)
    assert np.all(np.abs(got - ref.ce.row_loss)[valid] <= tol[valid])
    assert np.all(got[~valid] == 0.0)
    zl = out["z_loss"].cpu().numpy().astype(np.float64)
    z_tol = 2 * 2e-3 * (np.abs(z).max(axis=1) + 7) * dz.max(axis=1) + 1e-5 * np.abs(ref.ce.z_loss)
    assert np.all((np.abs(zl - ref.ce.z_loss) <= z_tol)[valid])
    gh = _f64(out["grad_hidden"])
    assert np.all(gh[~valid] == 0.0)
    assert np.max(np.abs(gh - ref.grad_hidden)) <= 0.05 * np.abs(ref.grad_hidden).max()
    gw = out["grad_weight"].cpu().numpy().astype(np.float64)
    assert np.max(np.abs(gw - ref.grad_weight)) <= 0.05 * np.abs(ref.grad_weight).max()


@pytest.mark.parametrize("reduction", ["mean", "none"])
def test_flce_no_host_sync(reduction):
    """flce_forward_backward under torch's sync debug mode "error": the
    compaction's count and every normalizer stay on the device."""
    h, W, t, cw = _problem(16, 200, 128, 640, weighted=True)
    dev = h.device
    tt = torch.from_numpy(t).to(dev)
    cwt = torch.from_numpy(cw).to(dev)
    go = torch.full((200,), 0.5, device=dev) if reduction == "none" else \
        torch.tensor(0.5, device=dev)
    torch.cuda.synchronize()
    torch.cuda.set_sync_debug_mode("error")
    try:
        out = vf.flce_forward_backward(h, W, tt, cwt, -100, 0.1, reduction, chunk_rows=64,
                                       grad_output=go)
    finally:
        torch.cuda.set_sync_debug_mode("default")
    torch.cuda.synchronize()
    ref = oracle.flce(_f64(h), _f64(W), t, cw.astype(np.float64), -100, 0.1, reduction,
                      0.5 if reduction != "none" else np.full(200, 0.5))
    gw = out["grad_weight"].cpu().numpy().astype(np.float64)
    assert np.max(np.abs(gw - ref.grad_weight)) <= 0.05 * np.abs(ref.grad_weight).max()


def test_flce_graph_capture_replays_match_eager():
    """The whole FLCE captured in a HIP graph: every replay (with eager work
    and synchronizations in between) equals the eager result bit for bit."""
    h, W, t, _ = _problem(17, 300, 128, 1000)
    dev = h.device
    tt = torch.from_numpy(t).to(dev)
    eager = vf.flce_forward_backward(h, W, tt, None, -100, 0.1, "mean", chunk_rows=128)
    torch.cuda.synchronize()
    e_loss, e_gh, e_gw = (eager["loss"].clone(), eager["grad_hidden"].clone(),
                          eager["grad_weight"].clone())
    ws = eager["workspace"]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        vf.flce_forward_backward(h, W, tt, None, -100, 0.1, "mean", chunk_rows=128,
                                 workspace=ws)  # warm-up
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        res = vf.flce_forward_backward(h, W, tt, None, -100, 0.1, "mean", chunk_rows=128,
                                       workspace=ws)
    for _ in range(3):
        res["grad_weight"].fill_(7.0)
        res["grad_hidden"].fill_(7.0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(res["loss"], e_loss)
        assert torch.equal(res["grad_hidden"], e_gh)
        assert torch.equal(res["grad_weight"], e_gw)
        _ = (h.float() * 2).sum()  # unrelated eager work between replays


def test_flce_empty_batch():
    """No rows: the mean is NaN (0/0), dL/dW is zero, nothing else is written."""
    dev = _dev()
    rng = np.random.default_rng(18)
    h = torch.empty((0, 128), dtype=torch.bfloat16, device=dev)
    W = _bf16(rng, (300, 128), 0.2, dev)
    t = torch.empty(0, dtype=torch.int64, device=dev)
    out = vf.flce_forward_backward(h, W, t, None, -100, 0.0, "mean")
    torch.cuda.synchronize()
    assert np.isnan(float(out["loss"]))
    assert torch.all(out["grad_weight"] == 0)


def test_flce_one_class():
    """V = 1: the loss and both gradients are 0 (the softmax of one logit is
    1); the row takes the per-element path of the cross-entropy."""
    dev = _dev()
    rng = np.random.default_rng(19)
    h = _bf16(rng, (40, 64), 1.0, dev)
    W = _bf16(rng, (1, 64), 1.0, dev)
    t = torch.zeros(40, dtype=torch.int64, device=dev)
    out = vf.flce_forward_backward(h, W, t, None, -100, 0.1, "sum", row_loss=True)
    torch.cuda.synchronize()
    assert float(out["loss"]) == 0.0
    assert torch.all(out["row_loss"] == 0)
    assert torch.all(out["grad_hidden"] == 0) and torch.all(out["grad_weight"] == 0)


def test_flce_bad_target_is_flagged():
    """A target outside [0, V) that is not ignore_index: kept by the
    compaction so the cross-entropy flags it (status bit, NaN row loss, zero
    gradient row), and the mean is NaN."""
    h, W, t, _ = _problem(20, 64, 128, 256, ignore_frac=0.1)
    t = t.copy()
    t[5] = 256 + 7
    dev = h.device
    out = vf.flce_forward_backward(h, W, torch.from_numpy(t).to(dev), None, -100, 0.0, "mean",
                                   row_loss=True)
    torch.cuda.synchronize()
    st = vf.status(out["workspace"])
    assert st["status"] & 1 and st["n_invalid"] == 1
    assert np.isnan(float(out["loss"]))
    rl = out["row_loss"].cpu().numpy()
    assert np.isnan(rl[5]) and np.all(np.isfinite(np.delete(rl, 5)))
    assert torch.all(out["grad_hidden"][5] == 0)
    # the other rows' gradients are those of the batch without row 5 and
    # with W = the valid count (the bad row is out of the mean)
    keep = np.ones(64, bool)
    keep[5] = False
    ref = oracle.flce(_f64(h)[keep], _f64(W), t[keep], None, -100, 0.0, "mean")
    gh = _f64(out["grad_hidden"])[keep]
    assert np.max(np.abs(gh - ref.grad_hidden)) <= 0.05 * np.abs(ref.grad_hidden).max()


# ---------------------------------------------------------------- the autograd wrapper

def test_linear_cross_entropy_autograd_mean():
    """loss.backward(0.5): the gradients equal the FLCE's with grad_output 0.5
    bit for bit (a power-of-two scale commutes with every rounding), dL/dW
    cast by autograd to the weight's bf16."""
    from vocab_softmax_cross_amd import linear_cross_entropy
    h, W, t, cw = _problem(21, 200, 128, 640, weighted=True)
    dev = h.device
    tt = torch.from_numpy(t).to(dev)
    cwt = torch.from_numpy(cw).to(dev)
    hg = h.clone().requires_grad_(True)
    Wg = W.clone().requires_grad_(True)
    loss = linear_cross_entropy(hg, Wg, tt, cwt, -100, 0.1, "mean")
    loss.backward(torch.tensor(0.5, device=dev))
    ref = vf.flce_forward_backward(h, W, tt, cwt, -100, 0.1, "mean",
                                   grad_output=torch.tensor(0.5, device=dev))
    torch.cuda.synchronize()
    assert float(loss) == float(ref["loss"])
    assert torch.equal(hg.grad, ref["grad_hidden"])
    assert torch.equal(Wg.grad, ref["grad_weight"].to(torch.bfloat16))
    with pytest.raises(RuntimeError):
        loss2 = linear_cross_entropy(h.clone().requires_grad_(True), W, tt, None)
        loss2.backward(retain_graph=True)
        loss2.backward()


def test_linear_cross_entropy_autograd_none_per_row():
    from vocab_softmax_cross_amd import linear_cross_entropy
    h, W, t, _ = _problem(22, 150, 64, 512)
    dev = h.device
    tt = torch.from_numpy(t).to(dev)
    go = torch.linspace(0.1, 2.0, 150, device=dev)
    hg = h.clone().requires_grad_(True)
    Wg = W.clone().requires_grad_(True)
    loss = linear_cross_entropy(hg, Wg, tt, None, -100, 0.0, "none", chunk_rows=64)
    loss.backward(go)
    ref = vf.flce_forward_backward(h, W, tt, None, -100, 0.0, "none", chunk_rows=64,
                                   grad_output=go)
    torch.cuda.synchronize()
    assert torch.equal(loss.detach(), ref["loss"])
    assert torch.equal(hg.grad, ref["grad_hidden"])
    assert torch.equal(Wg.grad, ref["grad_weight"].to(torch.bfloat16))
