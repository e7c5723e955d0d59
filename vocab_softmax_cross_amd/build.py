"""Builds libvsce.so (the HIP kernels and the C ABI of include/vsce.h) in-tree.

Every translation unit under csrc/ is compiled for gfx950 with hipcc, in
parallel, and linked into ``vocab_softmax_cross_amd/libvsce.so``.

    python -m vocab_softmax_cross_amd.build          # build
    python -m vocab_softmax_cross_amd.build --asm    # also keep the gfx950 assembly
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import os
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


def _compile(src: str, keep_asm: bool) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    if keep_asm:
        cmd.append(f"--save-temps=obj")
    r = subprocess.run(cmd, cwd=BUILD, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    msg = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{msg}")
    if msg.strip():
        print(msg, file=sys.stderr)
    return obj


def build(keep_asm: bool = False, jobs: int | None = None, verbose: bool = True) -> str:
    """Compile every source and link libvsce.so; returns the library path."""
    os.makedirs(BUILD, exist_ok=True)
    jobs = jobs or min(len(SOURCES), max(1, min(16, os.cpu_count() or 1)))
    with cf.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, keep_asm), SOURCES))
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
