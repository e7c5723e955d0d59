"""The C ABI on the host: the library loads, exports what include/vsce.h
declares, and rejects invalid arguments before any HIP call (CPU only: no
call here reaches a kernel launch)."""
import ctypes
import os
import re

import pytest

import vocab_softmax_cross_amd._lib as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "vsce.h")

FAKE = 0x10000  # a 256-byte-aligned address that is never dereferenced


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^[A-Za-z_][\w\s\*]*?\b(\w+)\s*\([^;{]*\)\s*;", text, flags=re.M)
    return sorted(set(n for n in names if not n.startswith("__")))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("ce_forward_fused_inplace", "ce_forward_stats", "ce_backward_from_stats",
              "ce_scale_grad", "vsce_workspace_bytes"):
        assert n in names


def test_library_exports_every_declared_symbol():
    lib = L.load()
    for n in declared_functions():
        assert hasattr(lib, n), n
    assert set(declared_functions()) == set(L.EXPORTS)


def test_version_and_workspace_size():
    assert L.vsce_version() >= 200
    assert L.vsce_workspace_bytes(-1) == 0
    assert L.vsce_workspace_bytes(0) == L.WS_HEADER_BYTES
    # header, then [rows] fp32 scratch for row losses, accuracies and z-losses,
    # and [rows] float4 statistics of the fused mode's rows read twice
    assert L.vsce_workspace_bytes(1) == L.WS_HEADER_BYTES + 4 * 256
    assert L.vsce_workspace_bytes(8192) == L.WS_HEADER_BYTES + 3 * 8192 * 4 + 8192 * 16


def test_header_constants_match_the_binding():
    text = open(HEADER).read()
    defines = {m.group(1): int(m.group(2), 0)
               for m in re.finditer(r"^#define\s+VSCE_(\w+)\s+(0x[0-9a-fA-F]+|\d+)u?\b", text,
                                    flags=re.M)}
    for name in ("WS_W", "WS_SUM_W", "WS_N_VALID", "WS_N_INVALID", "WS_STATUS", "WS_INV_W",
                 "WS_INV_N_VALID", "WS_HEADER_BYTES", "STATS_STRIDE", "PARTIAL_STRIDE",
                 "FLAG_LONG_ROWS_RING", "NOALLOC_MAX_ROWS"):
        assert defines[name] == getattr(L, name), name


def test_struct_layout_matches_the_header():
    assert ctypes.sizeof(L.Problem) == 88
    assert L.Problem.label_smoothing.offset == 56
    assert L.Problem.softcap.offset == 60
    assert L.Problem.z_loss.offset == 64
    assert L.Problem.flags.offset == 68
    assert L.Problem.vocab_offset.offset == 72
    assert L.Problem.vocab_total.offset == 80
    assert ctypes.sizeof(L.Outputs) == 40
    assert L.Outputs.z_loss.offset == 32
    # the header declares the fields in the same order
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    body = re.search(r"typedef struct vsce_problem \{(.*?)\}", text, re.S).group(1)
    names = re.findall(r"(\w+)\s*;", body)
    assert names == [f[0] for f in L.Problem._fields_]
    body = re.search(r"typedef struct vsce_outputs \{(.*?)\}", text, re.S).group(1)
    assert re.findall(r"(\w+)\s*;", body) == [f[0] for f in L.Outputs._fields_]


def _problem(**kw):
    p = L.Problem()
    p.rows, p.vocab, p.row_stride = 8, 64, 64
    p.dtype, p.reduction = L.BF16, L.REDUCTION_MEAN
    p.target, p.class_weight = FAKE, None
    p.ignore_index, p.label_smoothing, p.flags = -100, 0.0, 0
    p.softcap, p.z_loss = 0.0, 0.0
    p.vocab_offset, p.vocab_total = 0, 0
    for k, v in kw.items():
        setattr(p, k, v)
    return p


def _outputs(loss=FAKE):
    o = L.Outputs()
    o.loss = loss
    return o


def _fused(p, logits=FAKE, out="default", ws=FAKE):
    o = _outputs() if out == "default" else out
    return L.raw_call("ce_forward_fused_inplace", None if p is None else ctypes.byref(p), logits,
                      None if o is None else ctypes.byref(o), ws, None)


def _stats(p, stats=FAKE, logits=FAKE, ws=FAKE):
    return L.raw_call("ce_forward_stats", ctypes.byref(p), logits, stats,
                      ctypes.byref(_outputs()), ws, None)


@pytest.mark.parametrize("field,value", [
    ("rows", -1), ("vocab", 0), ("vocab", -3), ("row_stride", 63), ("dtype", 3), ("dtype", -1),
    ("reduction", 3), ("flags", 2), ("flags", 0x80000001), ("label_smoothing", -0.1),
    ("label_smoothing", 1.5),
    ("label_smoothing", float("nan")), ("target", None),
    ("softcap", -1.0), ("softcap", float("nan")), ("softcap", float("inf")),
    ("z_loss", -1e-4), ("z_loss", float("nan")), ("z_loss", float("inf")),
])
def test_bad_problem_fields_are_rejected(field, value):
    assert _fused(_problem(**{field: value})) == L.ERR_INVALID
    assert _stats(_problem(**{field: value})) == L.ERR_INVALID


def test_bad_pointers_are_rejected():
    assert _fused(None) == L.ERR_INVALID
    assert _fused(_problem(), logits=None) == L.ERR_INVALID
    assert _fused(_problem(), logits=FAKE + 1) == L.ERR_INVALID      # bf16 needs 2-byte alignment
    assert _fused(_problem(dtype=L.F32), logits=FAKE + 2) == L.ERR_INVALID
    assert _fused(_problem(), out=None) == L.ERR_INVALID
    assert _fused(_problem(), out=_outputs(loss=None)) == L.ERR_INVALID
    assert _fused(_problem(), ws=None) == L.ERR_INVALID
    assert _fused(_problem(), ws=FAKE + 8) == L.ERR_INVALID           # workspace: 256-byte aligned
    assert _fused(_problem(class_weight=FAKE + 2)) == L.ERR_INVALID
    assert _stats(_problem(), stats=None) == L.ERR_INVALID
    assert _stats(_problem(), stats=FAKE + 4) == L.ERR_INVALID


def _partial(p, logits=FAKE, partial=FAKE):
    return L.raw_call("ce_forward_stats_partial", ctypes.byref(p), logits, partial, None)


def _merge(p, partials=FAKE, shards=2, stats=FAKE, out="default", ws=FAKE):
    o = _outputs() if out == "default" else out
    return L.raw_call("ce_merge_stats", ctypes.byref(p), partials, shards, stats,
                      None if o is None else ctypes.byref(o), ws, None)


@pytest.mark.parametrize("offset,total", [(-1, 128), (65, 128), (0, 63), (8, 64)])
def test_bad_vocab_shards_are_rejected(offset, total):
    p = _problem(vocab_offset=offset, vocab_total=total)
    assert _partial(p) == L.ERR_INVALID
    assert _backward(p) == L.ERR_INVALID


def test_whole_row_entry_points_refuse_a_shard():
    p = _problem(vocab_offset=64, vocab_total=128)
    assert _fused(p) == L.ERR_INVALID
    assert _stats(p) == L.ERR_INVALID
    assert _merge(p) == L.ERR_INVALID


def test_partial_and_merge_argument_checks():
    shard = _problem(vocab_offset=64, vocab_total=128)
    assert _partial(shard, partial=None) == L.ERR_INVALID
    assert _partial(shard, partial=FAKE + 4) == L.ERR_INVALID       # 16-byte records
    assert _partial(_problem(rows=0, vocab_offset=64, vocab_total=128), partial=None) == L.OK
    full = _problem(vocab=128, row_stride=128)
    assert _merge(full, shards=0) == L.ERR_INVALID
    assert _merge(full, partials=None) == L.ERR_INVALID
    assert _merge(full, stats=FAKE + 8) == L.ERR_INVALID
    assert _merge(full, out=None) == L.ERR_INVALID
    assert _merge(full, ws=FAKE + 8) == L.ERR_INVALID


def test_unsupported_sizes():
    assert _fused(_problem(vocab=1 << 30, row_stride=1 << 30)) == L.ERR_UNSUPPORTED
    assert _fused(_problem(rows=1 << 31)) == L.ERR_UNSUPPORTED


def _backward(p, grad=FAKE, stats=FAKE, go=FAKE, go_stride=0, ws=FAKE):
    return L.raw_call("ce_backward_from_stats", ctypes.byref(p), FAKE, grad, stats, go, go_stride,
                      ws, None)


def test_backward_argument_checks():
    assert _backward(_problem(), grad=None) == L.ERR_INVALID
    assert _backward(_problem(), grad=FAKE + 1) == L.ERR_INVALID
    assert _backward(_problem(), stats=None) == L.ERR_INVALID
    assert _backward(_problem(), go=None) == L.ERR_INVALID
    assert _backward(_problem(), go_stride=2) == L.ERR_INVALID
    assert _backward(_problem(), ws=None) == L.ERR_INVALID
    assert _backward(_problem(vocab=0)) == L.ERR_INVALID
    # nothing to do for an empty batch: accepted without touching the GPU
    assert _backward(_problem(rows=0), grad=None, stats=None, go=None) == L.OK


def _scale(grad=FAKE, rows=4, vocab=64, stride=64, dtype=L.BF16, go=FAKE, go_stride=0):
    return L.raw_call("ce_scale_grad", grad, rows, vocab, stride, dtype, go, go_stride, 1, None)


def test_scale_argument_checks():
    assert _scale(dtype=7) == L.ERR_INVALID
    assert _scale(rows=-1) == L.ERR_INVALID
    assert _scale(vocab=0) == L.ERR_INVALID
    assert _scale(stride=10) == L.ERR_INVALID
    assert _scale(go_stride=-1) == L.ERR_INVALID
    assert _scale(grad=None) == L.ERR_INVALID
    assert _scale(go=None) == L.ERR_INVALID
    assert _scale(grad=FAKE + 1) == L.ERR_INVALID
    assert _scale(rows=0, grad=None, go=None) == L.OK


def test_strerror():
    lib = L.load()
    assert lib.vsce_strerror(L.ERR_INVALID) == b"invalid argument"
    assert lib.vsce_strerror(12345) == b"unknown error"


def test_binding_raises_on_error_codes():
    with pytest.raises(L.VsceError) as e:
        L.ce_forward_fused_inplace(_problem(vocab=0), FAKE, _outputs(), FAKE, 0)
    assert e.value.code == L.ERR_INVALID


# ---------------------------------------------------------------- FLCE and its GEMM

def test_flce_problem_layout_matches_the_header():
    assert ctypes.sizeof(L.FlceProblem) == 72
    assert L.FlceProblem.target.offset == 32
    assert L.FlceProblem.label_smoothing.offset == 56
    assert L.FlceProblem.reduction.offset == 68
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    body = re.search(r"typedef struct vsce_flce_problem \{(.*?)\}", text, re.S).group(1)
    assert re.findall(r"(\w+)\s*;", body) == [f[0] for f in L.FlceProblem._fields_]


def _flce_problem(**kw):
    p = L.FlceProblem()
    p.rows, p.hidden, p.vocab, p.chunk_rows = 100, 128, 1000, 0
    p.target, p.class_weight, p.ignore_index = FAKE, None, -100
    p.label_smoothing, p.softcap, p.z_loss, p.reduction = 0.0, 0.0, 0.0, L.REDUCTION_MEAN
    for k, v in kw.items():
        setattr(p, k, v)
    return p


def _flce(p, hidden=FAKE, weight=FAKE, out="default", go=None, go_stride=0, gh=FAKE, gw=FAKE,
          ws=FAKE):
    o = _outputs() if out == "default" else out
    return L.raw_call("flce_forward_backward", ctypes.byref(p), hidden, weight,
                      None if o is None else ctypes.byref(o), go, go_stride, gh, gw, ws, None)


def test_flce_workspace_size():
    # one chunk's logits (their gradient in place), compacted hidden states
    # and their gradient, per-row scratch; no transposed copies (the products
    # read W, G and h k-major)
    p = _flce_problem(rows=8192, hidden=4096, vocab=128256)
    b = L.vsce_flce_workspace_bytes(p)
    assert b >= 2 * 8192 * 128256 + 2 * 2 * 8192 * 4096
    assert b < 2 * 8192 * 128256 + 2 * 2 * 8192 * 4096 + 16e6
    chunked = L.vsce_flce_workspace_bytes(_flce_problem(rows=8192, hidden=4096, vocab=128256,
                                                        chunk_rows=1024))
    assert chunked < b - 1.5e9  # the logits of one chunk only
    assert L.vsce_flce_workspace_bytes(_flce_problem(hidden=100)) == 0


@pytest.mark.parametrize("field,value", [("rows", -1), ("hidden", 100), ("hidden", 0),
                                         ("vocab", 0), ("chunk_rows", -5), ("reduction", 4),
                                         ("label_smoothing", 2.0), ("softcap", -1.0),
                                         ("z_loss", float("nan")), ("target", None)])
def test_flce_bad_problem_fields_are_rejected(field, value):
    assert _flce(_flce_problem(**{field: value})) == L.ERR_INVALID


def test_flce_bad_pointers_are_rejected():
    p = _flce_problem()
    assert _flce(p, weight=None) == L.ERR_INVALID
    assert _flce(p, gw=None) == L.ERR_INVALID
    assert _flce(p, ws=None) == L.ERR_INVALID
    assert _flce(p, ws=FAKE + 16) == L.ERR_INVALID    # 256-byte aligned workspace
    assert _flce(p, hidden=FAKE + 2) == L.ERR_INVALID  # 16-byte aligned operands
    assert _flce(p, gh=None) == L.ERR_INVALID
    assert _flce(p, out=None) == L.ERR_INVALID
    assert _flce(p, out=_outputs(loss=None)) == L.ERR_INVALID
    assert _flce(p, go=FAKE, go_stride=2) == L.ERR_INVALID


def _gemm(M=128, N=128, K=64, lda=64, ldb=64, ldc=128, mode=0, A=FAKE, B=FAKE, C=FAKE):
    return L.raw_call("vsce_gemm_bf16_nt", A, lda, B, ldb, C, ldc, M, N, K, mode, None)


@pytest.mark.parametrize("kw", [dict(K=96, lda=96, ldb=96), dict(lda=32), dict(ldb=40),
                                dict(lda=68), dict(N=126, ldc=128), dict(ldc=126),
                                dict(ldc=64), dict(mode=3), dict(M=-1), dict(A=FAKE + 8),
                                dict(C=None), dict(lda=(1 << 23) + 8, ldb=64),
                                dict(lda=1 << 23), dict(ldb=1 << 23),
                                dict(ldc=(1 << 22) + 4), dict(ldc=(1 << 21) + 4, mode=1)])
def test_gemm_argument_checks(kw):
    assert _gemm(**kw) == L.ERR_INVALID


def _gemm_l(layout, M=128, N=128, K=64, lda=64, ldb=64, ldc=128, mode=0):
    return L.raw_call("vsce_gemm_bf16", FAKE, lda, FAKE, ldb, FAKE, ldc, M, N, K, layout, mode,
                      None)


@pytest.mark.parametrize("kw", [dict(layout=4), dict(layout=1, M=128, lda=120),
                                dict(layout=2, N=128, ldb=96), dict(layout=1, lda=132),
                                dict(layout=3, lda=1 << 23, ldb=128),
                                dict(layout=0, lda=32)])
def test_gemm_layout_argument_checks(kw):
    """k-major operands need a leading dimension of at least M (A) or N (B),
    a multiple of 8 below 2^23; unknown layout bits are rejected."""
    assert _gemm_l(**kw) == L.ERR_INVALID


def test_gemm_empty_is_a_no_op():
    assert _gemm(M=0) == L.OK
    assert _gemm(N=0) == L.OK


# ---------------------------------------------------------------- which HIP runtime the library binds
# PyTorch ships its own HIP and HSA runtimes with the same sonames as the
# system ROCm's; the library must bind to the copy torch uses.  Each case runs
# in a fresh interpreter, because a process keeps whatever it has loaded.

_MAPS = r"""
import sys
def runtimes():
    found = set()
    for line in open("/proc/self/maps"):
        p = line.split()[-1]
        if "libamdhip64" in p or "libhsa-runtime64" in p:
            found.add(p)
    return sorted(found)
"""


def _run(code):
    import subprocess
    import sys
    r = subprocess.run([sys.executable, "-c", _MAPS + code], cwd=ROOT, capture_output=True,
                       text=True, timeout=300)
    assert r.returncode == 0, r.stderr
    return [l for l in r.stdout.splitlines() if l.startswith("/")]


def test_load_binds_the_library_to_torchs_runtime():
    """_lib.load() alone, in a fresh process: one HIP runtime and one HSA
    runtime are mapped, both torch's."""
    maps = _run("import vocab_softmax_cross_amd._lib as L\nL.load()\n"
                "import torch\nprint('\\n'.join(runtimes()))")
    hip = [p for p in maps if "libamdhip64" in p]
    hsa = [p for p in maps if "libhsa-runtime64" in p]
    assert len(hip) == 1 and len(hsa) == 1, maps
    assert "torch" in hip[0] and "torch" in hsa[0], maps


@pytest.mark.skipif(os.path.exists("/dev/kfd"), reason="hosts without a GPU only: the order "
                    "shown here puts two HIP runtimes over one device")
def test_loading_the_library_before_torch_maps_two_runtimes():
    """The order load() rules out: the library opened with a bare dlopen before
    torch is imported maps the system ROCm runtime, and torch then maps its
    own as well (no HIP call is made; nothing touches a device)."""
    maps = _run(f"import ctypes\nctypes.CDLL({L.LIB_PATH!r})\n"
                "import torch\nprint('\\n'.join(runtimes()))")
    assert len([p for p in maps if "libamdhip64" in p]) == 2, maps


def test_noalloc_rejects_more_rows_than_its_static_workspace():
    """The check happens before any HIP call (no GPU needed)."""
    lib = L.load()
    p = L.Problem()
    p.rows, p.vocab, p.row_stride, p.dtype, p.reduction = L.NOALLOC_MAX_ROWS + 1, 1024, 1024, \
        L.BF16, L.REDUCTION_MEAN
    p.target, p.ignore_index = FAKE, -100
    out = L.Outputs()
    out.loss = FAKE
    assert L.raw_call("ce_forward_fused_inplace_noalloc", ctypes.byref(p), FAKE,
                      ctypes.byref(out), None) == L.ERR_TOO_LARGE
    assert lib.vsce_strerror(L.ERR_TOO_LARGE) == b"more rows than the static workspace holds"
    # argument errors still come first
    p.vocab = 0
    assert L.raw_call("ce_forward_fused_inplace_noalloc", ctypes.byref(p), FAKE,
                      ctypes.byref(out), None) == L.ERR_INVALID
    # the static array holds the workspace of the largest accepted problem
    assert L.vsce_workspace_bytes(L.NOALLOC_MAX_ROWS) < 2 << 20
