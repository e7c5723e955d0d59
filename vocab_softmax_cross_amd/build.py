"""Builds libvsce.so (the HIP kernels and the C ABI of include/vsce.h) in-tree.

Every translation unit under csrc/ is compiled for gfx950 with hipcc, in
parallel, and linked into ``vocab_softmax_cross_amd/libvsce.so``.  The
compiler's per-kernel resource report (registers, spills, scratch, occupancy)
is written to _build/kernel_resources.txt, and a kernel that spills to scratch
without a reason listed in SCRATCH_ALLOWED fails the build.

    python -m vocab_softmax_cross_amd.build          # build
    python -m vocab_softmax_cross_amd.build --asm    # also keep the gfx950 assembly
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import os
import re
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libvsce.so")

SOURCES = [
    "abi.hip",
    "small.hip",
    "stream_f32.hip",
    "stream_bf16.hip",
    "stream_f16.hip",
    "stream_f32_cap.hip",
    "stream_bf16_cap.hip",
    "stream_f16_cap.hip",
    "fused_f32.hip",
    "fused_bf16.hip",
    "fused_f16.hip",
    "fused_f32_cap.hip",
    "fused_bf16_cap.hip",
    "fused_f16_cap.hip",
    "gemm.hip",
    "flce.hip",
]

# Kernels allowed to use scratch memory (register spills), each with its
# reason.  Keys are fused_resident_kernel shapes (threads, register slots, LDS
# slots, overflow slots, weighted, capped) over every element type; any other
# kernel whose compiled ScratchSize is nonzero fails the build.
SCRATCH_ALLOWED = {
    (1024, 11, 5, 0, True, False):
        "class weights on the two-rows-per-CU shape (rows of at most 16320 vectors): each "
        "vector's 8 weights stay in flight beside the 44 row registers",
    (1024, 11, 5, 0, True, True):
        "class weights and a soft-cap on the two-rows-per-CU shape: the weights in flight "
        "and the cap's slope beside the 44 row registers",
}

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    # No packed fp32 instructions (v_pk_{add,mul,fma}_f32) in device code.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE,
]
RESOURCE_REMARKS = "-Rpass-analysis=kernel-resource-usage"
REPORT = os.path.join(BUILD, "kernel_resources.txt")


def _resources(text: str) -> tuple[list[dict], str]:
    """The compiler's per-kernel resource remarks, and the rest of its output."""
    kernels, rest, cur = [], [], None
    lines = text.splitlines()
    i = 0
    while i < len(lines):
        line = lines[i]
        if RESOURCE_REMARKS in line:
            m = re.search(r"remark:\s+(.*?):?\s+(\S+) \[" + re.escape(RESOURCE_REMARKS), line)
            key, val = (m.group(1), m.group(2)) if m else (None, None)
            if key == "Function Name":
                cur = {"name": val}
                kernels.append(cur)
            elif cur is not None and key:
                cur[key] = val
            # the remark's source excerpt (two lines) follows it
            while i + 1 < len(lines) and re.match(r"^\s+(\d+ )?\|", lines[i + 1]):
                i += 1
        elif not line.startswith("In file included from"):
            rest.append(line)
        i += 1
    return kernels, "\n".join(rest)


def _compile(src: str, keep_asm: bool):
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, RESOURCE_REMARKS, "-c", os.path.join(CSRC, src), "-o", obj]
    if keep_asm:
        cmd.append(f"--save-temps=obj")
    r = subprocess.run(cmd, cwd=BUILD, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    kernels, other = _resources(r.stdout + r.stderr)
    msg = "\n".join(l for l in other.splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{msg}")
    if msg.strip():
        print(msg, file=sys.stderr)
    for k in kernels:
        k["source"] = src
    return obj, kernels


_SHAPE = re.compile(r"fused_resident_kernelILi(\d)ELi(\d+)ELi(\d+)ELi(\d+)ELi(\d+)ELi(\d+)"
                    r"ELb(\d)ELb(\d)ELi(\d+)E")


def scratch_reason(name: str):
    """The listed reason a kernel may use scratch, or None."""
    m = _SHAPE.search(name)
    if not m:
        return None
    _, nt, nreg, nlds, _, nov, w, cap, _ = (int(g) for g in m.groups())
    return SCRATCH_ALLOWED.get((nt, nreg, nlds, nov, bool(w), bool(cap)))


def check_resources(kernels: list[dict]) -> None:
    """Writes the per-kernel report and fails on scratch use outside
    SCRATCH_ALLOWED."""
    bad = []
    with open(REPORT, "w") as fh:
        fh.write("source kernel VGPRs AGPRs VGPR-spill SGPR-spill scratch[B/lane] waves/SIMD\n")
        for k in sorted(kernels, key=lambda k: (k["source"], k["name"])):
            scratch = int(k.get("ScratchSize [bytes/lane]", "0"))
            fh.write(f"{k['source']} {k['name']} {k.get('VGPRs')} {k.get('AGPRs')} "
                     f"{k.get('VGPRs Spill')} {k.get('SGPRs Spill')} {scratch} "
                     f"{k.get('Occupancy [waves/SIMD]')}\n")
            if scratch > 0 and scratch_reason(k["name"]) is None:
                bad.append(f"{k['source']}: {k['name']} uses {scratch} B/lane of scratch")
    if bad:
        raise RuntimeError("kernels spill to scratch without a listed reason "
                           "(SCRATCH_ALLOWED in build.py):\n" + "\n".join(bad))


def build(keep_asm: bool = False, jobs: int | None = None, verbose: bool = True) -> str:
    """Compile every source and link libvsce.so; returns the library path."""
    os.makedirs(BUILD, exist_ok=True)
    jobs = jobs or min(len(SOURCES), max(1, min(16, os.cpu_count() or 1)))
    with cf.ThreadPoolExecutor(jobs) as ex:
        results = list(ex.map(lambda s: _compile(s, keep_asm), SOURCES))
    objs = [o for o, _ in results]
    check_resources([k for _, ks in results for k in ks])
    tmp = LIB + f".tmp{os.getpid()}"
    r = subprocess.run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


def clean() -> None:
    shutil.rmtree(BUILD, ignore_errors=True)


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--asm", action="store_true", help="keep the gfx950 assembly under _build/")
    ap.add_argument("-j", "--jobs", type=int, default=None)
    args = ap.parse_args()
    build(keep_asm=args.asm, jobs=args.jobs)
