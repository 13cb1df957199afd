"""Build libqgemv.so (gfx950) in-tree with hipcc.

    python -m quantized_weight_gemv_amd.build [--isa DIR]

Each translation unit is compiled separately (in parallel) into _build/, then
linked into quantized_weight_gemv_amd/libqgemv.so.  ``--isa DIR`` also writes
the gfx950 assembly of every HIP source into DIR for inspection.
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
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libqgemv.so")
ARCH = "gfx950"

# Packed-FP32 instruction generation is switched off: only fp16 packed math is
# used on purpose, and fp32 code stays scalar.
COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-I", INCLUDE, "-I", CSRC,
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-Wno-unused-command-line-argument"]


def _hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


def sources() -> list[str]:
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith((".hip", ".cpp")))


def _compile(src: str, isa_dir: str | None) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [_hipcc(), *COMMON, "-c", src, "-o", obj]
    if src.endswith(".cpp"):
        cmd = [_hipcc(), "-x", "c++", "-O2", "-std=c++17", "-fPIC", "-I", INCLUDE, "-I", CSRC, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    if isa_dir and src.endswith(".hip"):
        os.makedirs(isa_dir, exist_ok=True)
        out = os.path.join(isa_dir, os.path.basename(src) + ".s")
        subprocess.run([_hipcc(), *COMMON, "--cuda-device-only", "-S", src, "-o", out], check=True,
                       capture_output=True)
    return obj


def build(isa_dir: str | None = None, verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources()
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda s: _compile(s, isa_dir), srcs))
    tmp = LIB + ".tmp"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--isa", default=None)
    a = ap.parse_args()
    build(a.isa, verbose=True)
    sys.exit(0)
