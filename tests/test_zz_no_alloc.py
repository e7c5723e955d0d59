"""ce_forward_fused_inplace_noalloc (the workspace taken from the library's
static per-device array) against ce_forward_fused_inplace with a caller's
workspace, through the C ABI: bit-identical gradients and loss outputs, on
calls in a row whose inputs shrink, so that each call runs over what the
previous one left in the static array."""

import numpy as np
import pytest
import torch

import oracle
import workloads as W
import vocab_softmax_cross_amd._lib as L
from tests.compare import assert_loss_close

pytestmark = pytest.mark.gpu

DT = {"f32": L.F32, "bf16": L.BF16, "f16": L.F16}


def _dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def _small(name, BT, V, **kw):
    d = dict(W.WORKLOADS[name].__dict__)
    d.update(BT=BT, V=V, **kw)
    return W.Workload(**d)


def _forward(entry, wl, x, t, wt, reduction, softcap, z_loss, dev):
    """One fused forward through `entry`; returns its loss outputs."""
    rows = wl.BT
    p = L.Problem()
    p.rows, p.vocab, p.row_stride = rows, wl.V, x.stride(0)
    p.dtype, p.reduction = DT[wl.dtype], L.REDUCTIONS[reduction]
    p.target = t.data_ptr()
    p.class_weight = None if wt is None else wt.data_ptr()
    p.ignore_index, p.label_smoothing, p.flags = -100, wl.label_smoothing, 0
    p.softcap, p.z_loss = softcap, z_loss
    res = {
        "loss": torch.full((rows if reduction == "none" else 1,), -1.0, device=dev),
        "row_loss": torch.full((rows,), -1.0, device=dev),
        "token_acc": torch.full((rows,), -1.0, device=dev),
        "acc_mean": torch.full((1,), -1.0, device=dev),
        "z_loss": torch.full((rows if reduction == "none" else 1,), -1.0, device=dev),
    }
    out = L.Outputs()
    for k, v in res.items():
        setattr(out, k, v.data_ptr())
    stream = torch.cuda.current_stream(dev).cuda_stream
    if entry == "noalloc":
        L.ce_forward_fused_inplace_noalloc(p, x.data_ptr(), out, stream)
    else:
        ws = torch.empty(L.vsce_workspace_bytes(rows), dtype=torch.uint8, device=dev)
        L.ce_forward_fused_inplace(p, x.data_ptr(), out, ws.data_ptr(), stream)
        res["_ws"] = ws
    return res


# Each sequence runs its calls in order; every call is smaller than the one
# before it.  (workload, rows, V, overrides, reduction, softcap, z_loss)
SEQUENCES = {
    "headline_then_long_rows": [
        ("llm_head", 512, 128256, {}, "mean", 0.0, 0.0),
        # rows too long for the chip: the statistics go to the static array
        ("llm_head", 8, 300000, {"ignore_frac": 0.25}, "none", 0.0, 0.0),
    ],
    "weighted_then_capped": [
        ("weighted", 96, 151936, {}, "sum", 0.0, 0.0),
        ("llm_head", 40, 32000, {}, "mean", 30.0, 1e-4),
    ],
}


@pytest.mark.parametrize("seq", list(SEQUENCES))
def test_noalloc_matches_the_workspace_entry_point(seq):
    dev = _dev()
    for name, rows, V, kw, reduction, softcap, z_loss in SEQUENCES[seq]:
        wl = _small(name, rows, V, **kw)
        print(f"[case] noalloc {seq}: {name} BT={rows} V={V} {reduction} softcap={softcap} "
              f"z_loss={z_loss}", flush=True)
        tgt = W.targets(wl)
        w = W.class_weights(wl)
        xh = W.logits(wl, tgt)
        t = torch.from_numpy(tgt).to(dev)
        wt = None if w is None else torch.from_numpy(w).to(dev)
        got, ref = {}, {}
        for entry, store in (("noalloc", got), ("workspace", ref)):
            x = xh.to(dev)
            store.update(_forward(entry, wl, x, t, wt, reduction, softcap, z_loss, dev))
            store["grad"] = x
        torch.cuda.synchronize()
        assert torch.equal(got["grad"], ref["grad"]), "gradient differs"
        for k in ("loss", "row_loss", "token_acc", "acc_mean", "z_loss"):
            a, b = got[k].cpu().numpy(), ref[k].cpu().numpy()
            np.testing.assert_array_equal(a, b, err_msg=k)
        # and the loss against the oracle, at the loss bar
        r = oracle.cross_entropy(W.as_f64(xh), tgt, w, -100, wl.label_smoothing, reduction,
                                 1.0, None, want_grad=False, softcap=softcap, z_loss=z_loss)
        assert_loss_close(got["loss"].cpu().numpy().astype(np.float64), r.loss)
