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
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-fhip-fp32-correctly-rounded-divide-sqrt",
          "-Wno-unused-command-line-argument"]


def _hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


def sources() -> list[str]:
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith((".hip", ".cpp")))


def _compile(src: str, isa_dir: str | None, defines=(), build_dir: str = BUILD) -> str:
    obj = os.path.join(build_dir, os.path.basename(src) + ".o")
    cmd = [_hipcc(), *COMMON, *[f"-D{d}" for d in defines], "-c", src, "-o", obj]
    if src.endswith(".cpp"):
        cmd = [_hipcc(), "-x", "c++", "-O2", "-std=c++17", "-fPIC", "-I", INCLUDE, "-I", CSRC, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    if isa_dir and src.endswith(".hip"):
        os.makedirs(isa_dir, exist_ok=True)
        out = os.path.join(isa_dir, os.path.basename(src) + ".s")
        subprocess.run([_hipcc(), *COMMON, *[f"-D{d}" for d in defines], "--cuda-device-only", "-S", src,
                        "-o", out], check=True, capture_output=True)
    return obj


def build(isa_dir: str | None = None, verbose: bool = False, defines=(), out: str | None = None) -> str:
    """Compile and link; ``defines`` / ``out`` build a variant elsewhere."""
    lib = out or LIB
    build_dir = BUILD if out is None else os.path.join(BUILD, "variant_" + "_".join(defines))
    os.makedirs(build_dir, exist_ok=True)
    srcs = sources()
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda s: _compile(s, isa_dir, defines, build_dir), srcs))
    tmp = lib + ".tmp"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib)
    if verbose:
        print(f"built {lib}")
    return lib


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--isa", default=None)
    ap.add_argument("-D", dest="defines", action="append", default=[])
    ap.add_argument("--out", default=None)
    a = ap.parse_args()
    build(a.isa, verbose=True, defines=a.defines, out=a.out)
    sys.exit(0)
