"""Build liblca.so (HIP kernels for gfx950 + the C ABI) in-tree with hipcc.

Usage: python -m long_context_attention_12_amd.build [--verbose]
"""

from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
OBJ = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "liblca.so")
SOURCES = ["compress.hip", "index_topk.hip", "attend.hip", "out_proj.hip", "lca_api.cpp"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # keep the compiler from forming packed fp32 (v_pk_*_f32) instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


# Per-source additions: MFMA results in VGPRs. The indexer's feed a short VALU
# epilogue per tile (no accumulator read per result register); the tiled
# projection's would otherwise move between the register files every K step.
EXTRA = {"index_topk.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
         "out_proj.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def _compile(src: str, verbose: bool) -> str:
    out = os.path.join(OBJ, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, *EXTRA.get(src, []), "-c", os.path.join(CSRC, src), "-o", out]
    if src.endswith(".cpp"):
        cmd = [HIPCC, "-x", "hip", *FLAGS, "-c", os.path.join(CSRC, src), "-o", out]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
    if verbose and r.stderr.strip():
        print(r.stderr, flush=True)
    return out


def build(verbose: bool = False) -> str:
    os.makedirs(OBJ, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(4, len(SOURCES))) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    build_validate_timing(verbose)
    return LIB


def build_validate_timing(verbose: bool = False) -> str:
    """The host-check timing loop (csrc/validate_timing.c), a plain C program
    linked against liblca.so; it runs without a GPU."""
    exe = os.path.join(OBJ, "validate_timing")
    cmd = ["gcc", "-O2", "-std=c11", "-Wall", os.path.join(CSRC, "validate_timing.c"),
           "-I", os.path.join(os.path.dirname(PKG), "include"), "-L", PKG, "-llca",
           "-Wl,-rpath," + PKG, "-o", exe]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"gcc failed on validate_timing.c:\n{r.stdout}\n{r.stderr}")
    return exe


if __name__ == "__main__":
    print(build(verbose="--verbose" in sys.argv))
