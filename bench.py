#!/usr/bin/env python3
"""Throughput of the fused softmax cross-entropy hot path on one MI355X.

One step = one forward + backward of the whole path over one batch through
the C ABI: the device-side normalizers, the fused row kernel (loss, accuracy
and the gradient written over the logits), the loss reduction, and the
grad_output scale (a no-op launch at grad_output = 1.0).  The default workload
is the LLM head: BT = 8192 rows of V = 128256 bf16 logits ~ N(0, 2), 5% of
rows ignored, label smoothing 0.1, mean reduction.

Each step gets its own freshly written copy of the logits (a ring of
pre-filled buffers in HBM), because the fused forward overwrites its input
with the gradient.  The run prints one JSON line:
  value      rows per second of whole fwd+bwd steps (wall clock over K steps,
             with nothing recorded inside the timed region)
  roofline   the row kernel alone: algorithmic bytes per launch / its mean
             launch time from HIP events recorded around that launch, in a
             second timed run of the same K steps
  cpu_baseline  the fp64 oracle on a bounded sample of the same rows
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0  # dense bf16 matrix-core peak
RING_CAP_BYTES = 120 << 30  # HBM for pre-filled logits copies
PROFILE = os.path.join(ROOT, "profiles", "traffic_fused_resident_llm_head.md")
KERNEL_SOURCES = ["common.h", "rowmath.h", "fused_impl.h", "fused_bf16.hip"]


def parse():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="llm_head")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra-modes", action="store_true",
                    help="skip the split-mode and grad_output != 1 context timings")
    ap.add_argument("--flce-only", action="store_true",
                    help="run only the FLCE measurement (a short run for profiling) and print "
                         "its JSON line")
    ap.add_argument("--only-workload", choices=("confidence", "weighted"),
                    help="run only the row kernel on that workload's full size (a short run for "
                         "profiling) and print its JSON line")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="oracle time budget for the cpu_baseline sample")
    return ap.parse_args()


class Hip:
    """The few HIP runtime calls the bench needs (events), via ctypes."""

    def __init__(self):
        self.lib = ctypes.CDLL("libamdhip64.so")
        self.lib.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.lib.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def event(self) -> int:
        e = ctypes.c_void_p()
        if self.lib.hipEventCreate(ctypes.byref(e)) != 0:
            raise RuntimeError("hipEventCreate failed")
        return e.value

    def elapsed_ms(self, a: int, b: int) -> float:
        ms = ctypes.c_float()
        if self.lib.hipEventElapsedTime(ctypes.byref(ms), a, b) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return float(ms.value)

    def destroy(self, e: int) -> None:
        self.lib.hipEventDestroy(e)

    def record(self, e: int, stream: int) -> None:
        if self.lib.hipEventRecord(ctypes.c_void_p(e), ctypes.c_void_p(stream)) != 0:
            raise RuntimeError("hipEventRecord failed")

    def launch_ms(self, fn, n: int, stream: int) -> float:
        """Median GPU time of one launch of fn() over n launches, each between
        its own pair of events on `stream` (host launch overhead excluded)."""
        import numpy as np
        evs = [(self.event(), self.event()) for _ in range(n)]
        for a, b in evs:
            self.record(a, stream)
            fn()
            self.record(b, stream)
        self.lib.hipDeviceSynchronize()
        ms = [self.elapsed_ms(a, b) for a, b in evs]
        for a, b in evs:
            self.destroy(a)
            self.destroy(b)
        return float(np.median(ms))


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "vocab_softmax_cross_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def stored_traffic(workload: str):
    """HBM bytes per launch of the row kernel from the committed rocprofv3
    counter summary, if it was taken on the current kernel sources."""
    if not os.path.exists(PROFILE):
        return None
    vals = {}
    with open(PROFILE) as fh:
        for line in fh:
            if line.startswith("traffic:"):
                for kv in line[len("traffic:"):].split():
                    k, _, v = kv.partition("=")
                    vals[k] = v
    if vals.get("workload") != workload or vals.get("kernel_sources") != kernel_source_hash():
        return None
    try:
        return float(vals["bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def cpu_baseline(wl, tgt, budget_s: float, threads: int = 0):
    """The oracle (fp64 forward + gradient + rounding) on consecutive row
    chunks until about `budget_s` of oracle time; rows per second.  `threads`
    = 0 uses every host core the OpenMP runtime sees."""
    import numpy as np
    import oracle
    import workloads as W
    default_threads = oracle.max_threads()
    oracle.set_threads(threads if threads > 0 else default_threads)
    chunk = 512 if threads != 1 else 64
    done, spent = 0, 0.0
    while done < wl.BT and spent < budget_s:
        r1 = min(wl.BT, done + chunk)
        x = W.as_f64(W.logits_rows(wl, done, r1, tgt))
        t0 = time.perf_counter()
        oracle.normalizer(tgt, wl.V, None)
        r = oracle.rows(x, tgt[done:r1], None, -100, wl.label_smoothing, want_grad=True)
        g = r.grad * (1.0 / max(1, int(np.sum(tgt != -100))))
        oracle.round_to(g, wl.dtype)
        spent += time.perf_counter() - t0
        done = r1
        del x, r, g
    cores = oracle.max_threads()
    oracle.set_threads(default_threads)
    return {"value": done / spent, "unit": "rows/s", "cores": cores,
            "kind": "oracle",
            "sample": f"first {done} of {wl.BT} rows ({done * wl.V:.3g} elements), fp64 "
                      f"forward + gradient + rounding to {wl.dtype}, {spent:.1f} s"}


def long_rows_mode(L, W, hip, dev, stream, K):
    """The fused mode on rows too long to keep on chip (the wide fp32
    workload, 8192 x 256000): each row is read twice and written once.  Both
    kernel choices are timed per launch by events on the launch stream, each
    launch on a fresh copy of the logits: the default pair (statistics, then
    the gradient in place) and the one-launch LDS ring."""
    import numpy as np
    import torch
    wl = W.WORKLOADS["wide_fp32"]
    tgt = W.targets(wl)
    pristine = W.logits(wl, tgt).to(dev)
    n_buf = 4
    bufs = [torch.empty_like(pristine) for _ in range(n_buf)]
    t = torch.from_numpy(tgt).to(dev)
    ws = torch.empty(L.vsce_workspace_bytes(wl.BT), dtype=torch.uint8, device=dev)
    loss = torch.empty(wl.BT, dtype=torch.float32, device=dev)
    outs = L.Outputs()
    outs.loss = loss.data_ptr()
    n_valid = int(np.sum((tgt >= 0) & (tgt < wl.V)))
    row = wl.V * wl.elem_bytes
    alg = 3 * n_valid * row + (wl.BT - n_valid) * row + 12 * wl.BT

    def problem(flags):
        p = L.Problem()
        p.rows, p.vocab, p.row_stride = wl.BT, wl.V, wl.V
        p.dtype, p.reduction = L.F32, L.REDUCTIONS[wl.reductions[0]]
        p.target, p.class_weight = t.data_ptr(), None
        p.ignore_index, p.label_smoothing, p.flags = -100, wl.label_smoothing, flags
        p.softcap, p.z_loss = 0.0, 0.0
        return p

    res = {"workload": wl.name, "shape": [wl.BT, wl.V], "logits": wl.dtype,
           "alg_bytes_per_launch": alg}
    for name, flags in (("pair", 0), ("ring", L.FLAG_LONG_ROWS_RING)):
        p = problem(flags)
        ms = []
        for r0 in range(0, K, n_buf):
            for b in bufs:
                b.copy_(pristine)
            torch.cuda.synchronize()
            evs = [(hip.event(), hip.event()) for _ in range(min(n_buf, K - r0))]
            for b, (e0, e1) in zip(bufs, evs):
                L.ce_forward_fused_inplace_timed(p, b.data_ptr(), outs, ws.data_ptr(), stream,
                                                 e0, e1)
            torch.cuda.synchronize()
            ms += [hip.elapsed_ms(a, b) for a, b in evs]
            for a, b in evs:
                hip.destroy(a)
                hip.destroy(b)
        m = float(np.median(ms))
        res[name] = {"ms": round(m, 4), "alg_GBps": round(alg / m / 1e6, 1),
                     "frac_of_hbm_peak": round(alg / m / 1e6 / HBM_PEAK_GBPS, 4)}
    del bufs, pristine
    torch.cuda.empty_cache()
    return res


def workload_modes(L, W, hip, dev, stream, K, names=("confidence", "weighted")):
    """The fused row kernel on the other workloads' full sizes: the
    confidence workload (4096 x 32000 bf16, targets at p = 0.9 / 0.99 / 0.999)
    and the weighted one (16384 x 151936 bf16, class weights, smoothing 0.1,
    5% ignored rows, sum).  Each launch on a fresh copy of the logits, timed
    by events on the launch stream around the row kernel (as the headline's
    roofline), its algorithmic bytes: a read of every valid row, a write of
    every row, 12 bytes per row."""
    import numpy as np
    import torch
    res = {}
    for name in names:
        wl = W.WORKLOADS[name]
        tgt = W.targets(wl)
        w = W.class_weights(wl)
        pristine = W.logits_device(wl, dev, tgt)
        n_buf = 4
        bufs = [torch.empty_like(pristine) for _ in range(n_buf)]
        t = torch.from_numpy(tgt).to(dev)
        wt = None if w is None else torch.from_numpy(w).to(dev)
        ws = torch.empty(L.vsce_workspace_bytes(wl.BT), dtype=torch.uint8, device=dev)
        red = wl.reductions[0]
        loss = torch.empty(wl.BT if red == "none" else 1, dtype=torch.float32, device=dev)
        outs = L.Outputs()
        outs.loss = loss.data_ptr()
        p = L.Problem()
        p.rows, p.vocab, p.row_stride = wl.BT, wl.V, wl.V
        p.dtype, p.reduction = L.BF16, L.REDUCTIONS[red]
        p.target, p.class_weight = t.data_ptr(), (None if wt is None else wt.data_ptr())
        p.ignore_index, p.label_smoothing, p.flags = -100, wl.label_smoothing, 0
        p.softcap, p.z_loss = 0.0, 0.0
        n_valid = int(np.sum((tgt >= 0) & (tgt < wl.V)))
        row = wl.V * wl.elem_bytes
        alg = n_valid * row + wl.BT * row + 12 * wl.BT
        ms = []
        for r0 in range(0, K, n_buf):
            for b in bufs:
                b.copy_(pristine)
            torch.cuda.synchronize()
            evs = [(hip.event(), hip.event()) for _ in range(min(n_buf, K - r0))]
            for b, (e0, e1) in zip(bufs, evs):
                L.ce_forward_fused_inplace_timed(p, b.data_ptr(), outs, ws.data_ptr(), stream,
                                                 e0, e1)
            torch.cuda.synchronize()
            ms += [hip.elapsed_ms(a, b) for a, b in evs]
            for a, b in evs:
                hip.destroy(a)
                hip.destroy(b)
        m = float(np.median(ms))
        res[name] = {"shape": [wl.BT, wl.V], "logits": wl.dtype, "weighted": w is not None,
                     "label_smoothing": wl.label_smoothing, "reduction": red,
                     "kernel_ms": round(m, 4), "rows_per_s": round(wl.BT / m * 1e3, 1),
                     "alg_bytes_per_launch": alg, "alg_GBps": round(alg / m / 1e6, 1),
                     "frac_of_hbm_peak": round(alg / m / 1e6 / HBM_PEAK_GBPS, 4)}
        del bufs, pristine
        torch.cuda.empty_cache()
    return res


def cpu_baseline_flce(sample):
    """The FLCE oracle (fp64: z = h W^T, the cross-entropy, G W and G^T h)
    on the first rows of the FLCE mode's own inputs; rows per second."""
    import numpy as np
    import oracle
    h, w, t = sample
    try:
        from threadpoolctl import threadpool_info
        cores = max((p.get("num_threads", 1) for p in threadpool_info()), default=1)
    except ImportError:
        cores = os.cpu_count()
    t0 = time.perf_counter()
    oracle.flce(h, w, t, None, -100, 0.1, "mean")
    spent = time.perf_counter() - t0
    return {"value": len(t) / spent, "unit": "rows/s", "cores": cores, "kind": "oracle",
            "sample": f"first {len(t)} rows of the FLCE mode's inputs (H={h.shape[1]}, "
                      f"V={w.shape[0]}), fp64 logits, cross-entropy and both gradients, "
                      f"{spent:.1f} s"}


def flce_mode(L, W, hip, dev, stream, K, sample_rows=0):
    """The linear head fused with the cross-entropy at the pages' FLCE size
    (BT=8192, H=4096, V=128256 bf16; the headline workload's targets, 410
    ignored rows, smoothing 0.1, mean): flce_forward_backward per call, and
    each of its three products alone.  Bound by the matrix cores: the
    algorithmic work is 3 products of 2 n H V flops over the n kept rows."""
    import numpy as np
    import torch
    import vocab_softmax_cross_amd.functional as vf
    wl = W.WORKLOADS["llm_head"]
    BT, H, V = wl.BT, 4096, wl.V
    g = torch.Generator(device=dev)
    g.manual_seed(20)
    hidden = torch.randn((BT, H), generator=g, device=dev).to(torch.bfloat16)
    weight = (torch.randn((V, H), generator=g, device=dev) * (2.0 / H ** 0.5)).to(torch.bfloat16)
    tgt = W.targets(wl)
    t = torch.from_numpy(tgt).to(dev)
    n = int(np.sum(tgt != -100))
    p = vf.flce_problem(hidden, weight, t, None, -100, wl.label_smoothing, "mean")
    ws = torch.empty(L.vsce_flce_workspace_bytes(p), dtype=torch.uint8, device=dev)
    gh = torch.empty_like(hidden)
    gw = torch.empty((V, H), dtype=torch.float32, device=dev)
    loss = torch.empty(1, dtype=torch.float32, device=dev)
    outs = L.Outputs()
    outs.loss = loss.data_ptr()

    def call():
        L.flce_forward_backward(p, hidden.data_ptr(), weight.data_ptr(), outs, None, 0,
                                gh.data_ptr(), gw.data_ptr(), ws.data_ptr(), stream)

    call()
    torch.cuda.synchronize()
    reps = max(3, min(K, 10))
    ms = hip.launch_ms(call, reps, stream)
    flops = 3 * 2.0 * n * H * V
    res = {"shape": {"BT": BT, "H": H, "V": V, "kept_rows": n}, "ms": round(ms, 3),
           "TFLOPs": round(flops / ms / 1e9, 1),
           "frac_of_bf16_mfma_peak": round(flops / ms / 1e9 / MFMA_BF16_PEAK_TFLOPS, 4)}
    # The three products alone, at the same shapes and operand layouts as in
    # the FLCE (W, G and h read k-major, in place, by the backward products;
    # a bf16 G of the right size: its values do not change the work).
    a = torch.empty((BT, V), dtype=torch.bfloat16, device=dev).normal_(generator=g)
    zl = torch.empty((BT, V), dtype=torch.bfloat16, device=dev)
    dh = torch.empty((BT, H), dtype=torch.bfloat16, device=dev)
    products = {
        "z=hW^T": lambda: vf.gemm_bf16_nt(hidden, weight, out=zl),
        "dh=GW": lambda: vf.gemm_bf16_nt(a, weight.t(), out=dh),
        "dW=G^Th": lambda: vf.gemm_bf16_nt(a.t(), hidden.t(), out=gw),
    }
    one = 2.0 * BT * H * V
    for name, fn in products.items():
        fn()
        torch.cuda.synchronize()
        t_ms = hip.launch_ms(fn, reps, stream)
        res[name] = {"ms": round(t_ms, 3), "TFLOPs": round(one / t_ms / 1e9, 1)}
    sample = None
    if sample_rows:  # the oracle's sample: the same rows and weights, upcast exactly
        sample = (hidden[:sample_rows].double().cpu().numpy(), weight.double().cpu().numpy(),
                  tgt[:sample_rows].copy())
    del a, zl, dh, ws, gw, gh, weight, hidden
    torch.cuda.empty_cache()
    return res, sample


def graph_steps(L, wl, ring, refill, problems, outs, ws, go, dt, dev, K, Wu):
    """The headline step captured in a HIP graph: K fused steps (forward in
    place + grad_output scale), each on its own ring buffer, recorded once
    through torch's graph capture and replayed after the ring is refilled.
    Reported beside the eager step (the headline): the difference is the
    host launch overhead between the step's four kernels."""
    import numpy as np
    import torch

    n = len(ring)

    def steps(stream, first, count):
        for i in range(first, first + count):
            b = ring[i % n]
            L.ce_forward_fused_inplace(problems[i % n], b.data_ptr(), outs, ws.data_ptr(), stream)
            L.ce_scale_grad(b.data_ptr(), wl.BT, wl.V, wl.V, dt, go.data_ptr(), 0, 1, stream)

    side = torch.cuda.Stream(device=dev)
    side.wait_stream(torch.cuda.current_stream(dev))
    refill()
    with torch.cuda.stream(side):
        steps(side.cuda_stream, 0, Wu)  # warm-up outside the capture
    torch.cuda.current_stream(dev).wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        steps(torch.cuda.current_stream(dev).cuda_stream, 0, K)
    walls = []
    for _ in range(3):
        refill()
        t0 = time.perf_counter()
        graph.replay()
        torch.cuda.synchronize()
        walls.append(time.perf_counter() - t0)
    del graph
    wall = float(np.median(walls))
    return {"steps_per_graph": K, "ms_per_step": round(wall / K * 1e3, 4),
            "rows_per_s": round(wl.BT * K / wall, 1),
            "replays_ms_per_step": [round(w / K * 1e3, 4) for w in walls]}


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path (rows shard "
              "across GPUs with no exchange, one process per GPU). Use --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import vocab_softmax_cross_amd._lib as L
    import workloads as W

    # Initialise the HIP runtime (through torch) before the library is loaded,
    # so that the library registers its kernels with a running runtime, the
    # order every test and smoke() use.
    dev = torch.device("cuda:0")
    torch.cuda.init()
    torch.empty(1, device=dev)
    torch.cuda.synchronize()
    L.load()
    if args.flce_only:
        res, _ = flce_mode(L, W, Hip(), dev, torch.cuda.current_stream(dev).cuda_stream,
                           args.steps)
        print(json.dumps({"flce": res}), flush=True)
        return
    if args.only_workload:
        res = workload_modes(L, W, Hip(), dev, torch.cuda.current_stream(dev).cuda_stream,
                             args.steps, names=(args.only_workload,))
        print(json.dumps(res), flush=True)
        return
    wl = W.WORKLOADS[args.workload]
    K, Wu = args.steps, args.warmup
    tgt = W.targets(wl)
    n_valid = int(np.sum((tgt >= 0) & (tgt < wl.V)))
    row_bytes = wl.V * wl.elem_bytes

    t0 = time.perf_counter()
    host = W.logits(wl, tgt)
    gen_s = time.perf_counter() - t0
    pristine = host.to(dev)
    del host
    ring_n = max(1, min(K + Wu, RING_CAP_BYTES // max(1, wl.BT * row_bytes)))
    ring = [torch.empty_like(pristine) for _ in range(ring_n)]

    def refill():
        for b in ring:
            b.copy_(pristine)
        torch.cuda.synchronize()

    t = torch.from_numpy(tgt).to(dev)
    w = W.class_weights(wl)
    wt = None if w is None else torch.from_numpy(w).to(dev)
    red = wl.reductions[0]
    ws = torch.empty(L.vsce_workspace_bytes(wl.BT), dtype=torch.uint8, device=dev)
    loss = torch.empty(wl.BT if red == "none" else 1, dtype=torch.float32, device=dev)
    stats = torch.empty((wl.BT, L.STATS_STRIDE), dtype=torch.float32, device=dev)
    go_one = torch.ones(1, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev).cuda_stream
    dt = {"f32": L.F32, "bf16": L.BF16, "f16": L.F16}[wl.dtype]

    def problem(buf, softcap=0.0, z_loss=0.0):
        p = L.Problem()
        p.rows, p.vocab, p.row_stride = wl.BT, wl.V, wl.V
        p.dtype, p.reduction = dt, L.REDUCTIONS[red]
        p.target = t.data_ptr()
        p.class_weight = None if wt is None else wt.data_ptr()
        p.ignore_index, p.label_smoothing, p.flags = -100, wl.label_smoothing, 0
        p.softcap, p.z_loss = softcap, z_loss
        return p

    problems = [problem(b) for b in ring]
    # the context mode with both optional features: a Gemma-style cap and a
    # PaLM-style z-loss weight
    CAP, ZL = 30.0, 1e-4
    problems_cap = [problem(b, CAP, ZL) for b in ring]
    outs = L.Outputs()
    outs.loss = loss.data_ptr()
    hip = Hip()
    ev = [(hip.event(), hip.event()) for _ in range(K)]

    def fused_steps(probs):
        def fused_step(i, go, timed_events=None):
            b = ring[i % ring_n]
            if timed_events is None:
                L.ce_forward_fused_inplace(probs[i % ring_n], b.data_ptr(), outs, ws.data_ptr(),
                                           stream)
            else:
                L.ce_forward_fused_inplace_timed(probs[i % ring_n], b.data_ptr(), outs,
                                                 ws.data_ptr(), stream, *timed_events)
            L.ce_scale_grad(b.data_ptr(), wl.BT, wl.V, wl.V, dt, go.data_ptr(),
                            1 if go.numel() > 1 else 0, 1, stream)
        return fused_step

    fused_step = fused_steps(problems)

    def split_step(i, go):
        b = ring[i % ring_n]
        L.ce_forward_stats(problems[i % ring_n], b.data_ptr(), stats.data_ptr(), outs,
                           ws.data_ptr(), stream)
        L.ce_backward_from_stats(problems[i % ring_n], b.data_ptr(), b.data_ptr(),
                                 stats.data_ptr(), go.data_ptr(), 1 if go.numel() > 1 else 0,
                                 ws.data_ptr(), stream)

    def timed(step_fn, go, events=None):
        refill()
        for i in range(Wu):
            step_fn(i, go)
        torch.cuda.synchronize()
        t_begin = time.perf_counter()
        for i in range(K):
            if events is not None:
                step_fn(Wu + i, go, events[i])
            else:
                step_fn(Wu + i, go)
        torch.cuda.synchronize()
        return time.perf_counter() - t_begin

    # The step as a caller runs it: no events inside the timed region (each
    # event recorded between two kernels adds a marker of about 6 us to the
    # stream).  The row kernel's launch time comes from a second timed run of
    # the same K steps with a pair of events around each row-kernel launch.
    wall = timed(fused_step, go_one)
    wall_evented = timed(fused_step, go_one, events=ev)
    kernel_ms = [hip.elapsed_ms(a, b) for a, b in ev]
    mean_kernel_s = float(np.mean(kernel_ms)) / 1e3

    # algorithmic bytes: valid rows read + write, ignored rows write only,
    # plus the int64 target and fp32 loss of every row
    kernel_bytes = (2 * n_valid + (wl.BT - n_valid)) * row_bytes + 12 * wl.BT
    step_bytes = kernel_bytes + 8 * wl.BT + 4 * wl.BT  # normalizer + reduction reads
    ms_per_step = wall / K * 1e3
    value = wl.BT * K / wall
    achieved = kernel_bytes / mean_kernel_s / 1e9

    extra = {}
    flce_sample = None
    if not args.no_extra_modes:
        go37 = torch.full((1,), 0.37, dtype=torch.float32, device=dev)
        w37 = timed(fused_step, go37)
        try:  # a context mode: a capture failure is reported, not fatal to the line
            extra["fused_graph"] = graph_steps(L, wl, ring, refill, problems, outs, ws, go_one,
                                               dt, dev, K, Wu)
        except RuntimeError as e:
            torch.cuda.synchronize()
            extra["fused_graph"] = {"error": str(e)[:200]}
        wsp = timed(split_step, go_one)
        # the scale pass reads and writes every row
        extra["fused_go0.37"] = {"ms_per_step": round(w37 / K * 1e3, 4),
                                 "rows_per_s": round(wl.BT * K / w37, 1),
                                 "alg_GBps": round((kernel_bytes + 2 * wl.BT * row_bytes) * K
                                                   / w37 / 1e9, 1)}
        extra["split_go1"] = {"ms_per_step": round(wsp / K * 1e3, 4),
                              "rows_per_s": round(wl.BT * K / wsp, 1),
                              "alg_GBps": round((3 * n_valid * row_bytes
                                                 + (wl.BT - n_valid) * row_bytes) * K
                                                / wsp / 1e9, 1)}
        # soft-capped logits and a z-loss: same bytes, more arithmetic per
        # element (the cap and its slope: one exp and one reciprocal each in
        # the sum and gradient passes)
        for a, b in ev:
            hip.destroy(a)
            hip.destroy(b)
        ev[:] = [(hip.event(), hip.event()) for _ in range(K)]
        wcap = timed(fused_steps(problems_cap), go_one)
        timed(fused_steps(problems_cap), go_one, events=ev)
        cap_kernel_s = float(np.mean([hip.elapsed_ms(a, b) for a, b in ev])) / 1e3
        # One rank of an 8-way vocab-parallel layout at its real shape: the
        # statistics of its [BT, V/8] slice, the merge of the 8 gathered
        # records (here stacked on one device), its slice's backward.
        P = 8
        Vs = wl.V // P
        shard = pristine[:, :Vs].contiguous()
        grad_shard = torch.empty_like(shard)
        parts = torch.empty((P, wl.BT, L.PARTIAL_STRIDE), dtype=torch.float32, device=dev)
        merged = torch.empty((wl.BT, L.STATS_STRIDE), dtype=torch.float32, device=dev)

        def shard_problem(width, offset, stride):
            p = problem(None)
            p.vocab, p.row_stride, p.vocab_offset, p.vocab_total = width, stride, offset, wl.V
            return p

        for s_ in range(P):  # every rank's record, so that the merge sees real data
            a0 = s_ * Vs
            b0 = wl.V if s_ == P - 1 else a0 + Vs
            L.ce_forward_stats_partial(shard_problem(b0 - a0, a0, wl.V),
                                       pristine[:, a0:b0].data_ptr(), parts[s_].data_ptr(), stream)
        rank_p = shard_problem(Vs, 0, Vs)
        full_p = problem(None)
        merge_ws = torch.empty_like(ws)
        t_stats = hip.launch_ms(lambda: L.ce_forward_stats_partial(
            rank_p, shard.data_ptr(), parts[0].data_ptr(), stream), K, stream)
        t_merge = hip.launch_ms(lambda: L.ce_merge_stats(
            full_p, parts.data_ptr(), P, merged.data_ptr(), outs, merge_ws.data_ptr(), stream),
            K, stream)
        t_bwd = hip.launch_ms(lambda: L.ce_backward_from_stats(
            rank_p, shard.data_ptr(), grad_shard.data_ptr(), merged.data_ptr(),
            go_one.data_ptr(), 0, merge_ws.data_ptr(), stream), K, stream)
        shard_row = Vs * wl.elem_bytes
        extra["vocab_parallel_8_one_rank"] = {
            "shard": [wl.BT, Vs],
            "stats_ms": round(t_stats, 4),
            "stats_GBps": round(n_valid * shard_row / t_stats / 1e6, 1),
            "merge_ms": round(t_merge, 4),
            "backward_ms": round(t_bwd, 4),
            "backward_GBps": round((n_valid + wl.BT) * shard_row / t_bwd / 1e6, 1),
            "rank_kernels_ms": round(t_stats + t_merge + t_bwd, 4)}
        extra["fused_long_rows"] = long_rows_mode(L, W, hip, dev, stream, K)
        extra["fused_other_workloads"] = workload_modes(L, W, hip, dev, stream, K)
        extra["flce"], flce_sample = flce_mode(L, W, hip, dev, stream, K,
                                               0 if args.no_cpu_baseline else 64)
        extra[f"fused_softcap{CAP:g}_zloss{ZL:g}"] = {
            "ms_per_step": round(wcap / K * 1e3, 4),
            "rows_per_s": round(wl.BT * K / wcap, 1),
            "kernel_ms": round(cap_kernel_s * 1e3, 4),
            "kernel_GBps": round(kernel_bytes / cap_kernel_s / 1e9, 1),
            "kernel_frac_of_hbm_peak": round(kernel_bytes / cap_kernel_s / 1e9 / HBM_PEAK_GBPS, 4)}

    # Practical ceiling: the runtime's own device-to-device copy of one
    # logits buffer (reads and writes the same bytes as the row kernel's
    # valid rows), timed over K copies.
    copy_src, copy_dst = pristine, ring[0]
    torch.cuda.synchronize()
    t_copy = time.perf_counter()
    for _ in range(K):
        copy_dst.copy_(copy_src)
    torch.cuda.synchronize()
    copy_s = (time.perf_counter() - t_copy) / K
    copy_ceiling = {"kind": "torch copy_ (device to device)", "bytes": 2 * wl.BT * row_bytes,
                    "ms": round(copy_s * 1e3, 4),
                    "GBps": round(2 * wl.BT * row_bytes / copy_s / 1e9, 1)}

    # Peak memory of one fused forward + backward through the autograd entry
    # point, beside the logits it overwrites (the pages' measure: the
    # gradient takes the logits' place, so the peak is one logits tensor).
    from vocab_softmax_cross_amd import cross_entropy
    xm = ring[0]
    xm.copy_(pristine)
    xm.requires_grad_(True)
    torch.cuda.synchronize()
    torch.cuda.reset_peak_memory_stats()
    base_alloc = torch.cuda.memory_allocated()
    loss_m = cross_entropy(xm, t, label_smoothing=wl.label_smoothing, reduction=red)
    loss_m.backward()
    torch.cuda.synchronize()
    extra_alloc = torch.cuda.max_memory_allocated() - base_alloc
    logits_bytes = wl.BT * row_bytes
    peak_memory = {"kind": "torch max_memory_allocated over one fused forward + backward "
                           "(the cross_entropy autograd function), beyond what was allocated before",
                   "logits_MB": round(logits_bytes / 1e6, 1),
                   "extra_bytes": int(extra_alloc),
                   "peak_MB_with_logits": round((logits_bytes + extra_alloc) / 1e6, 1)}
    del loss_m
    xm.grad = None
    xm.requires_grad_(False)

    for a, b in ev:
        hip.destroy(a)
        hip.destroy(b)

    cpu = cpu1 = cpu_flce = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(wl, tgt, args.cpu_seconds)
        cpu1 = cpu_baseline(wl, tgt, args.cpu_seconds / 3, threads=1)
        if flce_sample is not None:
            cpu_flce = cpu_baseline_flce(flce_sample)

    line = {
        "metric": "fwd+bwd rows/s and HBM GB/s (% of peak) at BT=8192, V=128256 bf16",
        "value": round(value, 1),
        "unit": "rows/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": Wu,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",  # arithmetic type; the logits buffer type is in config
        "data": "synthetic",
        "config": {"workload": wl.name, "BT": wl.BT, "V": wl.V, "logits": wl.dtype,
                   "label_smoothing": wl.label_smoothing, "ignored_rows": wl.BT - n_valid,
                   "reduction": red, "grad_output": 1.0, "mode": "fused in-place"},
        "step_GBps": round(step_bytes * K / wall / 1e9, 1),
        "step_pct_of_hbm_peak": round(100 * step_bytes * K / wall / 1e9 / HBM_PEAK_GBPS, 2),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                     "traffic": stored_traffic(wl.name), "traffic_unit": "bytes/launch",
                     "kernel": "fused_resident_kernel", "bytes_per_launch": kernel_bytes,
                     "mean_launch_ms": round(mean_kernel_s * 1e3, 4),
                     "scope": "the row kernel alone: HIP events around its launch",
                     "step_frac": round(step_bytes * K / wall / 1e9 / HBM_PEAK_GBPS, 4),
                     "step_scope": "the whole step by the wall clock: normalizers, row kernel, "
                                   "loss reduction, grad_output scale",
                     "evented_ms_per_step": round(wall_evented / K * 1e3, 4)},
        "modes": extra,
        "copy_ceiling": copy_ceiling,
        "peak_memory": peak_memory,
        "cpu_baseline": cpu,
        "cpu_baseline_1thread": cpu1,
        "cpu_baseline_flce": cpu_flce,
        "input_gen_s": round(gen_s, 1),
        "ring_buffers": ring_n,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
