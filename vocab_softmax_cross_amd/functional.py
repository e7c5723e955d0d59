"""PyTorch entry points over the C ABI: device memory and streams come from
torch, every step of the computation runs in libvsce.so's HIP kernels.

Two modes (the pages' two designs):

* ``fused``: Liger-Kernel PR #1268's fused kernel.  The forward writes the
  gradient over the logits buffer (so peak memory stays at one logits tensor,
  per the linkedin#1290 commit message); the backward scales it in place by
  grad_output through the raw kernel (no autograd version bump), returning at
  once when grad_output == 1.0 (Liger-Kernel PR #1622, SKIP_IF_ONE).  After the
  call the logits tensor holds the gradient.
* ``split``: TransformerEngine PR #2325's split.  The forward saves per-row
  statistics (m, d', x_y, S) and leaves the logits intact; the backward
  recomputes the gradient in fp32 from them and writes it in the input type.

Both modes take the logit soft-cap ``softcap`` (x -> s tanh(x / s) before the
loss reads the logits) and the z-loss weight ``z_loss`` (lambda lse^2 per
valid row), the two CE features Liger-Kernel PR #1268 lists beside class
weights and label smoothing.

Nothing here synchronizes with the host: the normalizers and the loss
reduction stay on the device.
"""
from __future__ import annotations

from typing import Optional

import torch

from . import _lib as L

_DTYPES = {torch.float32: L.F32, torch.bfloat16: L.BF16, torch.float16: L.F16}


def _stream(t: torch.Tensor) -> int:
    return torch.cuda.current_stream(t.device).cuda_stream


def _rows_view(logits: torch.Tensor) -> torch.Tensor:
    """[..., V] -> a [rows, V] view with unit class stride (no copy)."""
    if logits.dim() < 2:
        raise ValueError("logits must have shape [..., V]")
    if logits.stride(-1) != 1:
        raise ValueError("logits must be contiguous along the class dimension")
    if logits.dim() == 2:
        return logits
    return logits.view(-1, logits.shape[-1])


def make_problem(x2d: torch.Tensor, target: torch.Tensor, weight: Optional[torch.Tensor],
                 ignore_index: int, label_smoothing: float, reduction: str,
                 softcap: float = 0.0, z_loss: float = 0.0, vocab_offset: int = 0,
                 vocab_total: int = 0) -> L.Problem:
    if x2d.dtype not in _DTYPES:
        raise TypeError(f"unsupported logits dtype {x2d.dtype}")
    if target.dtype != torch.int64 or target.device != x2d.device:
        raise TypeError("target must be an int64 tensor on the logits' device")
    if not target.is_contiguous() or target.numel() != x2d.shape[0]:
        raise ValueError("target must be contiguous with one entry per row")
    V = vocab_total or x2d.shape[1]
    if weight is not None:
        if weight.dtype != torch.float32 or not weight.is_contiguous() or weight.numel() != V:
            raise ValueError("class weights must be a contiguous float32 [V] tensor "
                             "(all V of them for a vocabulary shard)")
    p = L.Problem()
    p.rows = x2d.shape[0]
    p.vocab = x2d.shape[1]
    p.row_stride = x2d.stride(0) if x2d.shape[0] > 1 else x2d.shape[1]
    p.dtype = _DTYPES[x2d.dtype]
    p.reduction = L.REDUCTIONS[reduction]
    p.target = target.data_ptr() or None
    p.class_weight = None if weight is None else weight.data_ptr()
    p.ignore_index = int(ignore_index)
    p.label_smoothing = float(label_smoothing)
    p.softcap = float(softcap)
    p.z_loss = float(z_loss)
    p.flags = 0
    p.vocab_offset = int(vocab_offset)
    p.vocab_total = int(vocab_total)
    return p


def workspace_for(rows: int, device) -> torch.Tensor:
    return torch.empty(L.vsce_workspace_bytes(rows), dtype=torch.uint8, device=device)


def _outputs(rows: int, reduction: str, device, row_loss: bool, accuracy: bool,
             z_loss: bool = False):
    f32 = dict(dtype=torch.float32, device=device)
    per_row = max(rows, 1)
    loss = torch.empty(per_row if reduction == "none" else 1, **f32)
    rl = torch.empty(per_row, **f32) if row_loss else None
    acc = torch.empty(per_row, **f32) if accuracy else None
    accm = torch.empty(1, **f32) if accuracy else None
    zl = torch.empty(per_row if reduction == "none" else 1, **f32) if z_loss else None
    o = L.Outputs()
    o.loss = loss.data_ptr()
    o.row_loss = None if rl is None else rl.data_ptr()
    o.token_acc = None if acc is None else acc.data_ptr()
    o.acc_mean = None if accm is None else accm.data_ptr()
    o.z_loss = None if zl is None else zl.data_ptr()
    res = {
        "loss": loss[:rows] if reduction == "none" else loss[0],
        "row_loss": None if rl is None else rl[:rows],
        "token_acc": None if acc is None else acc[:rows],
        "acc_mean": None if accm is None else accm[0],
        "z_loss": None if zl is None else (zl[:rows] if reduction == "none" else zl[0]),
    }
    return o, res


def forward_fused_inplace(logits: torch.Tensor, target: torch.Tensor,
                          weight: Optional[torch.Tensor] = None, ignore_index: int = -100,
                          label_smoothing: float = 0.0, reduction: str = "mean",
                          row_loss: bool = False, accuracy: bool = False,
                          workspace: Optional[torch.Tensor] = None, softcap: float = 0.0,
                          z_loss: float = 0.0, return_z_loss: bool = False,
                          long_rows_ring: bool = False) -> dict:
    """ce_forward_fused_inplace: loss outputs; the logits buffer now holds the
    gradient of the reduced loss for grad_output = 1.  long_rows_ring sets
    VSCE_FLAG_LONG_ROWS_RING (one launch for rows too long for the chip)."""
    x = _rows_view(logits)
    p = make_problem(x, target.reshape(-1), weight, ignore_index, label_smoothing, reduction,
                     softcap, z_loss)
    p.flags = L.FLAG_LONG_ROWS_RING if long_rows_ring else 0
    ws = workspace if workspace is not None else workspace_for(p.rows, x.device)
    o, res = _outputs(p.rows, reduction, x.device, row_loss, accuracy, return_z_loss)
    L.ce_forward_fused_inplace(p, x.data_ptr(), o, ws.data_ptr(), _stream(x))
    res["workspace"] = ws
    return res


def forward_stats(logits: torch.Tensor, target: torch.Tensor,
                  weight: Optional[torch.Tensor] = None, ignore_index: int = -100,
                  label_smoothing: float = 0.0, reduction: str = "mean",
                  row_loss: bool = False, accuracy: bool = False,
                  workspace: Optional[torch.Tensor] = None, softcap: float = 0.0,
                  z_loss: float = 0.0, return_z_loss: bool = False) -> dict:
    """ce_forward_stats: loss outputs plus the [rows, 4] statistics."""
    x = _rows_view(logits)
    p = make_problem(x, target.reshape(-1), weight, ignore_index, label_smoothing, reduction,
                     softcap, z_loss)
    ws = workspace if workspace is not None else workspace_for(p.rows, x.device)
    stats = torch.empty((max(p.rows, 1), L.STATS_STRIDE), dtype=torch.float32, device=x.device)
    o, res = _outputs(p.rows, reduction, x.device, row_loss, accuracy, return_z_loss)
    L.ce_forward_stats(p, x.data_ptr(), stats.data_ptr(), o, ws.data_ptr(), _stream(x))
    res["stats"] = stats[:p.rows]
    res["workspace"] = ws
    return res


def _grad_output(go: torch.Tensor, rows: int, reduction: str, device):
    go = go.detach()
    if go.device != device:
        raise ValueError("grad_output must live on the logits' device")
    go = go.to(torch.float32).reshape(-1).contiguous()
    if go.numel() == 1:
        return go, 0
    if reduction == "none" and go.numel() == rows:
        return go, 1
    raise ValueError("grad_output must be a scalar or hold one value per row")


def backward_from_stats(logits: torch.Tensor, target: torch.Tensor, stats: torch.Tensor,
                        grad_output: torch.Tensor, workspace: torch.Tensor,
                        weight: Optional[torch.Tensor] = None, ignore_index: int = -100,
                        label_smoothing: float = 0.0, reduction: str = "mean",
                        out: Optional[torch.Tensor] = None, softcap: float = 0.0,
                        z_loss: float = 0.0, vocab_offset: int = 0,
                        vocab_total: int = 0) -> torch.Tensor:
    """ce_backward_from_stats: the gradient in the logits' type (``out`` may be
    the logits themselves for an in-place backward).  For one shard of a
    vocab-parallel layout pass its ``vocab_offset``, the full ``vocab_total``,
    the merged ``stats`` and the merge's workspace."""
    x = _rows_view(logits)
    p = make_problem(x, target.reshape(-1), weight, ignore_index, label_smoothing, reduction,
                     softcap, z_loss, vocab_offset, vocab_total)
    g = (torch.empty_strided(x.size(), x.stride(), dtype=x.dtype, device=x.device)
         if out is None else _rows_view(out))
    if g.shape != x.shape or g.dtype != x.dtype or g.stride() != x.stride():
        raise ValueError("out must match the logits' shape, dtype and strides")
    go, stride = _grad_output(grad_output, p.rows, reduction, x.device)
    L.ce_backward_from_stats(p, x.data_ptr(), g.data_ptr(), stats.data_ptr(), go.data_ptr(),
                             stride, workspace.data_ptr(), _stream(x))
    return g.view(logits.shape) if out is None else out


def forward_stats_partial(logits_shard: torch.Tensor, target: torch.Tensor, vocab_offset: int,
                          vocab_total: int, weight: Optional[torch.Tensor] = None,
                          ignore_index: int = -100, label_smoothing: float = 0.0,
                          softcap: float = 0.0,
                          out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """ce_forward_stats_partial: one vocabulary shard's per-row record
    ([rows, 8] fp32; see include/vsce.h).  ``logits_shard`` holds columns
    [vocab_offset, vocab_offset + width) of a ``vocab_total``-column
    vocabulary; targets are global; ``weight`` holds all vocab_total weights.
    ``out`` may be a slice of a stacked [shards, rows, 8] buffer."""
    x = _rows_view(logits_shard)
    p = make_problem(x, target.reshape(-1), weight, ignore_index, label_smoothing, "none",
                     softcap, 0.0, vocab_offset, vocab_total)
    part = out if out is not None else torch.empty((max(p.rows, 1), L.PARTIAL_STRIDE),
                                                    dtype=torch.float32, device=x.device)
    L.ce_forward_stats_partial(p, x.data_ptr(), part.data_ptr(), _stream(x))
    return part[:p.rows]


def merge_stats(partials: torch.Tensor, target: torch.Tensor, vocab_total: int,
                weight: Optional[torch.Tensor] = None, ignore_index: int = -100,
                label_smoothing: float = 0.0, reduction: str = "mean", softcap: float = 0.0,
                z_loss: float = 0.0, row_loss: bool = False, accuracy: bool = False,
                return_z_loss: bool = False, dtype: torch.dtype = torch.bfloat16) -> dict:
    """ce_merge_stats: the shards' stacked records ([shards, rows, 8], column
    order) -> the full rows' statistics, the loss outputs and the workspace,
    as ce_forward_stats gives them for the unsharded matrix."""
    if partials.dim() != 3 or partials.shape[2] != L.PARTIAL_STRIDE or not partials.is_contiguous():
        raise ValueError("partials must be a contiguous [shards, rows, 8] float32 tensor")
    shards, rows = partials.shape[0], partials.shape[1]
    dev = partials.device
    t = target.reshape(-1)
    if t.dtype != torch.int64 or t.device != dev or not t.is_contiguous() or t.numel() != rows:
        raise ValueError("target must be a contiguous int64 tensor with one entry per row")
    if weight is not None and (weight.dtype != torch.float32 or not weight.is_contiguous()
                               or weight.numel() != vocab_total):
        raise ValueError("class weights must be a contiguous float32 [vocab_total] tensor")
    p = L.Problem()
    p.rows, p.vocab, p.row_stride = rows, vocab_total, vocab_total  # no logits are read
    p.dtype, p.reduction = _DTYPES[dtype], L.REDUCTIONS[reduction]
    p.target = t.data_ptr() or None
    p.class_weight = None if weight is None else weight.data_ptr()
    p.ignore_index, p.label_smoothing = int(ignore_index), float(label_smoothing)
    p.softcap, p.z_loss, p.flags = float(softcap), float(z_loss), 0
    p.vocab_offset, p.vocab_total = 0, int(vocab_total)
    ws = workspace_for(rows, dev)
    stats = torch.empty((max(rows, 1), L.STATS_STRIDE), dtype=torch.float32, device=dev)
    o, res = _outputs(rows, reduction, dev, row_loss, accuracy, return_z_loss)
    L.ce_merge_stats(p, partials.data_ptr(), shards, stats.data_ptr(), o, ws.data_ptr(),
                     torch.cuda.current_stream(dev).cuda_stream)
    res["stats"] = stats[:rows]
    res["workspace"] = ws
    return res


def scale_grad(grad: torch.Tensor, grad_output: torch.Tensor, reduction: str = "mean",
               skip_if_one: bool = True) -> torch.Tensor:
    """ce_scale_grad: grad <- grad * grad_output in place (skipped where it is 1.0)."""
    g = _rows_view(grad)
    rows, V = g.shape
    go, stride = _grad_output(grad_output, rows, reduction, g.device)
    L.ce_scale_grad(g.data_ptr(), rows, V, g.stride(0) if rows > 1 else V, _DTYPES[g.dtype],
                    go.data_ptr(), stride, 1 if skip_if_one else 0, _stream(g))
    return grad


def _returns(res: dict, ctx, return_z_loss: bool, accuracy: bool):
    out = [res["loss"]]
    extra = []
    if return_z_loss:
        extra.append(res["z_loss"])
    if accuracy:
        extra += [res["token_acc"], res["acc_mean"]]
    if extra:
        ctx.mark_non_differentiable(*extra)
        return tuple(out + extra)
    return res["loss"]


class FusedCrossEntropy(torch.autograd.Function):
    """Fused mode: gradient computed in the forward, over the logits buffer."""

    @staticmethod
    def forward(ctx, logits, target, weight, ignore_index, label_smoothing, reduction, accuracy,
                softcap, z_loss, return_z_loss):
        res = forward_fused_inplace(logits, target, weight, ignore_index, label_smoothing,
                                    reduction, accuracy=accuracy, softcap=softcap, z_loss=z_loss,
                                    return_z_loss=return_z_loss)
        # The buffer now holds the gradient; it is written through raw pointers,
        # so autograd's version counter is untouched.
        ctx.save_for_backward(logits.detach())
        ctx.reduction = reduction
        ctx.grad_scaled_in_place = False
        ctx.workspace = res["workspace"]
        return _returns(res, ctx, return_z_loss, accuracy)

    @staticmethod
    def backward(ctx, grad_loss, *unused):
        if ctx.grad_scaled_in_place:
            raise RuntimeError("the fused cross-entropy gradient was already scaled in place; "
                               "a second backward (retain_graph=True) is not supported")
        ctx.grad_scaled_in_place = True
        (grad,) = ctx.saved_tensors
        scale_grad(grad, grad_loss, ctx.reduction, skip_if_one=True)
        return (grad,) + (None,) * 9


class SplitCrossEntropy(torch.autograd.Function):
    """Split mode: statistics in the forward, fp32 gradient in the backward."""

    @staticmethod
    def forward(ctx, logits, target, weight, ignore_index, label_smoothing, reduction, accuracy,
                inplace_backward, softcap, z_loss, return_z_loss):
        res = forward_stats(logits, target, weight, ignore_index, label_smoothing, reduction,
                            accuracy=accuracy, softcap=softcap, z_loss=z_loss,
                            return_z_loss=return_z_loss)
        ctx.save_for_backward(logits, target, res["stats"], res["workspace"],
                              *([] if weight is None else [weight]))
        ctx.args = (ignore_index, label_smoothing, reduction, weight is not None, inplace_backward,
                    softcap, z_loss)
        return _returns(res, ctx, return_z_loss, accuracy)

    @staticmethod
    def backward(ctx, grad_loss, *unused):
        logits, target, stats, ws, *w = ctx.saved_tensors
        ignore_index, ls, reduction, weighted, inplace, softcap, z_loss = ctx.args
        g = backward_from_stats(logits, target, stats, grad_loss, ws, w[0] if weighted else None,
                                ignore_index, ls, reduction,
                                out=logits.detach() if inplace else None, softcap=softcap,
                                z_loss=z_loss)
        return (g,) + (None,) * 10


def cross_entropy(logits: torch.Tensor, target: torch.Tensor, weight: Optional[torch.Tensor] = None,
                  ignore_index: int = -100, label_smoothing: float = 0.0,
                  reduction: str = "mean", *, mode: str = "fused", return_accuracy: bool = False,
                  inplace_backward: bool = False, softcap: float = 0.0, z_loss: float = 0.0,
                  return_z_loss: bool = False):
    """Softmax cross-entropy over the last dimension of ``logits``.

    ``mode="fused"`` overwrites ``logits`` with the gradient during the
    forward; ``mode="split"`` keeps them (and with ``inplace_backward`` writes
    the gradient over them in the backward).  ``softcap`` > 0 caps the logits
    at s tanh(x / s) first; ``z_loss`` > 0 adds lambda lse^2 per valid row
    (averaged over the valid rows under "mean").  Returns the loss, then the
    z-loss part when ``return_z_loss``, then the per-token accuracy and its
    mean over non-ignored rows when ``return_accuracy``; the extra outputs are
    not differentiable.
    """
    if reduction not in L.REDUCTIONS:
        raise ValueError(f"reduction must be one of {tuple(L.REDUCTIONS)}")
    if mode == "fused":
        return FusedCrossEntropy.apply(logits, target, weight, ignore_index, label_smoothing,
                                       reduction, return_accuracy, softcap, z_loss, return_z_loss)
    if mode == "split":
        return SplitCrossEntropy.apply(logits, target, weight, ignore_index, label_smoothing,
                                       reduction, return_accuracy, inplace_backward, softcap,
                                       z_loss, return_z_loss)
    raise ValueError("mode must be 'fused' or 'split'")


def status(workspace: torch.Tensor) -> dict:
    """Reads the workspace header (a device-to-host copy: synchronizes)."""
    h = workspace[:L.WS_HEADER_BYTES].cpu()
    return {
        "W": float(h[L.WS_W:L.WS_W + 8].view(torch.float64)[0]),
        "sum_w": float(h[L.WS_SUM_W:L.WS_SUM_W + 8].view(torch.float64)[0]),
        "n_valid": int(h[L.WS_N_VALID:L.WS_N_VALID + 8].view(torch.int64)[0]),
        "n_invalid": int(h[L.WS_N_INVALID:L.WS_N_INVALID + 8].view(torch.int64)[0]),
        "status": int(h[L.WS_STATUS:L.WS_STATUS + 4].view(torch.int32)[0]),
        "inv_W": float(h[L.WS_INV_W:L.WS_INV_W + 4].view(torch.float32)[0]),
        "inv_n_valid": float(h[L.WS_INV_N_VALID:L.WS_INV_N_VALID + 4].view(torch.float32)[0]),
    }


# ---------------------------------------------------------------- FLCE

def _operand(x: torch.Tensor, name: str):
    """(leading dimension, k-major) of a [rows, K] operand: contiguous along K
    (the row layout), else contiguous along its rows (a transposed view of a
    [K, rows] tensor, read k-major)."""
    if x.stride(1) == 1 or x.shape[1] == 1:
        return x.stride(0), False
    if x.stride(0) == 1 or x.shape[0] == 1:
        return x.stride(1), True
    raise ValueError(f"{name} must be contiguous along one of its dimensions")


def gemm_bf16_nt(a: torch.Tensor, b: torch.Tensor, out: Optional[torch.Tensor] = None,
                 accumulate: bool = False, out_dtype=torch.bfloat16) -> torch.Tensor:
    """vsce_gemm_bf16: a @ b.T for bf16 a [M, K] and b [N, K] on the matrix
    cores (K a multiple of 64); each operand contiguous along K or along its
    rows (e.g. g.t() for a [K, M] tensor g, read in place); bf16 or fp32 out,
    or added to an fp32 `out` when accumulate."""
    if a.dtype != torch.bfloat16 or b.dtype != torch.bfloat16 or a.dim() != 2 or b.dim() != 2:
        raise ValueError("a and b must be 2-D bfloat16 tensors")
    if a.shape[1] != b.shape[1]:
        raise ValueError("a and b must share K")
    lda, a_km = _operand(a, "a")
    ldb, b_km = _operand(b, "b")
    M, K = a.shape
    N = b.shape[0]
    if out is None:
        if accumulate:
            raise ValueError("accumulate needs an fp32 out")
        out = torch.empty((M, N), dtype=out_dtype, device=a.device)
    mode = (L.GEMM_OUT_F32_ADD if accumulate else L.GEMM_OUT_F32) \
        if out.dtype == torch.float32 else L.GEMM_OUT_BF16
    if out.dtype not in (torch.float32, torch.bfloat16) or out.shape != (M, N) or out.stride(1) != 1:
        raise ValueError("out must be a [M, N] float32 or bfloat16 tensor with contiguous rows")
    layout = (L.GEMM_A_K_MAJOR if a_km else 0) | (L.GEMM_B_K_MAJOR if b_km else 0)
    L.vsce_gemm_bf16(a.data_ptr(), lda, b.data_ptr(), ldb, out.data_ptr(), out.stride(0), M, N, K,
                     layout, mode, _stream(a))
    return out


def flce_problem(hidden: torch.Tensor, weight: torch.Tensor, target: torch.Tensor,
                 class_weight: Optional[torch.Tensor] = None, ignore_index: int = -100,
                 label_smoothing: float = 0.0, reduction: str = "mean", softcap: float = 0.0,
                 z_loss: float = 0.0, chunk_rows: int = 0):
    if hidden.dtype != torch.bfloat16 or weight.dtype != torch.bfloat16:
        raise ValueError("hidden and weight must be bfloat16")
    if hidden.dim() != 2 or weight.dim() != 2 or hidden.shape[1] != weight.shape[1]:
        raise ValueError("hidden [BT, H] and weight [V, H] must share H")
    if not hidden.is_contiguous() or not weight.is_contiguous():
        raise ValueError("hidden and weight must be contiguous")
    t = target.reshape(-1)
    if t.dtype != torch.int64 or not t.is_contiguous() or t.numel() != hidden.shape[0]:
        raise ValueError("target must be a contiguous int64 tensor with one entry per row")
    V = weight.shape[0]
    if class_weight is not None and (class_weight.dtype != torch.float32 or
                                     not class_weight.is_contiguous() or
                                     class_weight.numel() != V):
        raise ValueError("class weights must be a contiguous float32 [V] tensor")
    p = L.FlceProblem()
    p.rows, p.hidden, p.vocab, p.chunk_rows = hidden.shape[0], hidden.shape[1], V, int(chunk_rows)
    p.target = t.data_ptr() or None
    p.class_weight = None if class_weight is None else class_weight.data_ptr()
    p.ignore_index, p.label_smoothing = int(ignore_index), float(label_smoothing)
    p.softcap, p.z_loss, p.reduction = float(softcap), float(z_loss), L.REDUCTIONS[reduction]
    return p


def flce_forward_backward(hidden: torch.Tensor, weight: torch.Tensor, target: torch.Tensor,
                          class_weight: Optional[torch.Tensor] = None, ignore_index: int = -100,
                          label_smoothing: float = 0.0, reduction: str = "mean",
                          softcap: float = 0.0, z_loss: float = 0.0, chunk_rows: int = 0,
                          grad_output: Optional[torch.Tensor] = None, row_loss: bool = False,
                          accuracy: bool = False, return_z_loss: bool = False,
                          workspace: Optional[torch.Tensor] = None) -> dict:
    """flce_forward_backward: the loss outputs of cross_entropy(hidden @
    weight.T) and both gradients (grad_hidden bf16, grad_weight fp32)."""
    p = flce_problem(hidden, weight, target, class_weight, ignore_index, label_smoothing,
                     reduction, softcap, z_loss, chunk_rows)
    dev = hidden.device
    ws_bytes = L.vsce_flce_workspace_bytes(p)
    if ws_bytes == 0:
        raise ValueError("unsupported FLCE problem")
    ws = workspace if workspace is not None else torch.empty(ws_bytes, dtype=torch.uint8,
                                                              device=dev)
    if ws.numel() < ws_bytes:
        raise ValueError(f"workspace too small: {ws.numel()} < {ws_bytes} bytes")
    o, res = _outputs(p.rows, reduction, dev, row_loss, accuracy, return_z_loss)
    gh = torch.empty_like(hidden)
    gw = torch.empty(weight.shape, dtype=torch.float32, device=dev)
    go, go_stride = (None, 0) if grad_output is None else \
        _grad_output(grad_output, p.rows, reduction, dev)
    L.flce_forward_backward(p, hidden.data_ptr(), weight.data_ptr(), o,
                            None if go is None else go.data_ptr(), go_stride, gh.data_ptr(),
                            gw.data_ptr(), ws.data_ptr(), _stream(hidden))
    res["grad_hidden"], res["grad_weight"] = gh, gw
    res["workspace"] = ws
    return res


class LinearCrossEntropy(torch.autograd.Function):
    """The FLCE: loss of cross_entropy(hidden @ weight.T), both gradients
    computed in the forward (for grad_output 1) and scaled in place by the
    backward's scalar grad_output.  With reduction "none" and a grad_output
    per row, the backward runs the FLCE again with that grad_output (dL/dW
    mixes rows, so a per-row scale cannot be applied afterwards)."""

    @staticmethod
    def forward(ctx, hidden, weight, target, class_weight, ignore_index, label_smoothing,
                reduction, softcap, z_loss, chunk_rows):
        res = flce_forward_backward(hidden, weight, target, class_weight, ignore_index,
                                    label_smoothing, reduction, softcap, z_loss, chunk_rows)
        ctx.save_for_backward(hidden, weight, target,
                              *([] if class_weight is None else [class_weight]))
        ctx.args = (ignore_index, label_smoothing, reduction, softcap, z_loss, chunk_rows,
                    class_weight is not None)
        ctx.grads = (res["grad_hidden"], res["grad_weight"])
        ctx.used = False
        return res["loss"]

    @staticmethod
    def backward(ctx, grad_loss):
        if ctx.used:
            raise RuntimeError("the FLCE gradients were already scaled in place; a second "
                               "backward (retain_graph=True) is not supported")
        ctx.used = True
        ignore_index, ls, reduction, softcap, z_loss, chunk_rows, weighted = ctx.args
        gh, gw = ctx.grads
        ctx.grads = None
        if reduction == "none" and grad_loss.numel() > 1:
            hidden, weight, target, *cw = ctx.saved_tensors
            res = flce_forward_backward(hidden, weight, target, cw[0] if weighted else None,
                                        ignore_index, ls, reduction, softcap, z_loss,
                                        chunk_rows, grad_output=grad_loss)
            gh, gw = res["grad_hidden"], res["grad_weight"]
        else:
            scale_grad(gh, grad_loss.reshape(1), "mean", skip_if_one=True)
            scale_grad(gw, grad_loss.reshape(1), "mean", skip_if_one=True)
        return (gh, gw) + (None,) * 8


def linear_cross_entropy(hidden: torch.Tensor, weight: torch.Tensor, target: torch.Tensor,
                         class_weight: Optional[torch.Tensor] = None, ignore_index: int = -100,
                         label_smoothing: float = 0.0, reduction: str = "mean", *,
                         softcap: float = 0.0, z_loss: float = 0.0, chunk_rows: int = 0):
    """cross_entropy(hidden @ weight.T, target) without materialising more
    than one chunk of logits (bf16 hidden [BT, H] and weight [V, H]); autograd
    gives dL/dhidden (bf16) and dL/dweight (computed in fp32, cast by autograd
    to the weight's type)."""
    if reduction not in L.REDUCTIONS:
        raise ValueError(f"reduction must be one of {tuple(L.REDUCTIONS)}")
    return LinearCrossEntropy.apply(hidden, weight, target, class_weight, ignore_index,
                                    label_smoothing, reduction, softcap, z_loss, chunk_rows)
