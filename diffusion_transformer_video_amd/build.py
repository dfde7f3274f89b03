"""Build libdit.so (HIP kernels for gfx950 + the C-ABI layer) in-tree.

Every source is compiled with hipcc for gfx950 only; objects go to <repo>/_build
and the shared library lands next to this file, where the binding loads it.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OBJ = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libdit.so")

ARCH = "gfx950"
HIP_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17", "-Wall",
    # no packed-fp32 VALU forms: they are generated from plain float code otherwise
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


# Per-file extra flags. Attention never sees NaN inputs (finite scores, -inf only
# for masked keys), so IEEE-mode NaN quieting before every max is dropped there.
# The bf16 key loop is also scheduled with the memory-clause strategy and without
# the post-register-allocation reordering: same instructions, same results, and
# 2-3% faster (the exponentials spread evenly between the score products, K
# operand reads issued in pairs).
FILE_FLAGS = {
    "k_attn_bf16.hip": ["-fno-honor-nans", "-mno-amdgpu-ieee",
                        "-mllvm", "-amdgpu-sched-strategy=max-memory-clause",
                        "-mllvm", "-enable-post-misched=false"],
    "k_attn_fp8.hip": ["-fno-honor-nans", "-mno-amdgpu-ieee"],
}


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC)
                  if f.endswith((".hip", ".cpp")))


def _hipcc():
    h = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(h):
        raise RuntimeError("hipcc not found: the HIP toolchain is required to build libdit.so")
    return h


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(OBJ, os.path.basename(src) + ".o")
    cmd = [_hipcc(), *HIP_FLAGS, *FILE_FLAGS.get(os.path.basename(src), []), "-c", src, "-o", obj]
    if src.endswith(".cpp"):
        cmd[1:1] = ["-x", "hip"]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    msg = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                    if "packed-fp32-ops" not in l and l.strip())
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{msg}")
    if msg and verbose:
        print(msg, file=sys.stderr)
    return obj


def build(verbose: bool = False, jobs: int = 8) -> str:
    """Compile every source and link libdit.so; returns the library path."""
    os.makedirs(OBJ, exist_ok=True)
    srcs = sources()
    with cf.ThreadPoolExecutor(max_workers=max(1, min(jobs, len(srcs)))) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), srcs))
    tmp = LIB + ".tmp"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
