"""Build libpkv.so for gfx950 with hipcc (in-tree, next to this file).

    python -m paged_kv_cache_353_amd.build [--verbose] [--qk-valu]

--qk-valu builds the ablation library libpkv_qk_valu.so instead: the same
sources with q.K of the single-query decode on the VALU rather than the
matrix cores (bf16, head_dim 128), loaded in place of libpkv.so through
PKV_LIBRARY to measure what MFMA saves.
"""

from __future__ import annotations

import argparse
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libpkv.so")
QK_VALU_LIB = os.path.join(HERE, "libpkv_qk_valu.so")

SOURCES = ["kv_write.hip", "attn_decode.hip", "attn_multi.hip", "pkv_api.cpp"]
# Per-source extra flags.  The many-column kernel accumulates its output with
# MFMA and also scales it on the VALU; left to itself the compiler keeps the
# accumulators in AGPRs and copies them to and from VGPRs around every
# sub-tile.  The VGPR form of the MFMA instructions keeps them in one place.
EXTRA_FLAGS = {"attn_multi.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]}
ARCH = os.environ.get("PKV_OFFLOAD_ARCH", "gfx950")


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise FileNotFoundError("hipcc not found (set HIPCC or install ROCm)")


def compile_flags() -> list:
    return ["-O3", "-std=c++20", f"--offload-arch={ARCH}", "-fPIC", "-Wall",
            "-Wno-unused-function", "-munsafe-fp-atomics",
            # packed fp32 instructions are kept out of the generated code
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-I", INCLUDE, "-I", CSRC]


def _compile(src: str, verbose: bool, out_dir: str = BUILD_DIR, defines: tuple = ()) -> str:
    obj = os.path.join(out_dir, os.path.basename(src) + ".o")
    cmd = [hipcc()] + compile_flags() + EXTRA_FLAGS.get(src, []) + list(defines) + \
          ["-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compiling {src} failed:\n{r.stdout}\n{r.stderr}")
    noise = [ln for ln in r.stderr.splitlines() if "packed-fp32-ops" not in ln]
    if verbose and any(ln.strip() for ln in noise):
        print("\n".join(noise), file=sys.stderr)
    return obj


def build_library(verbose: bool = False, qk_valu: bool = False) -> str:
    """Compile every source and link libpkv.so (or, with qk_valu, the ablation
    library); always rebuilds."""
    out_dir = os.path.join(BUILD_DIR, "qk_valu") if qk_valu else BUILD_DIR
    lib = QK_VALU_LIB if qk_valu else LIB
    defines = ("-DPKV_QK_VALU=1",) if qk_valu else ()
    os.makedirs(out_dir, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose, out_dir, defines if s == "attn_decode.hip" else ()),
                           SOURCES))
    tmp = lib + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs + \
          ["-Wl,-soname,libpkv.so", "-Wl,--no-undefined"]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"linking libpkv.so failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib)
    return lib


def main() -> None:
    ap = argparse.ArgumentParser()
    ap.add_argument("--verbose", action="store_true")
    ap.add_argument("--qk-valu", action="store_true", help="build the VALU q.K ablation library instead")
    args = ap.parse_args()
    print(build_library(verbose=args.verbose, qk_valu=args.qk_valu))


if __name__ == "__main__":
    main()
