"""Build libtokengate.so (HIP kernels for gfx950 + the C ABI) in-tree with hipcc.

    python -m learned_token_pruning_mlp_amd.build

Every call recompiles every source; objects go to ``_build/`` (not committed).
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libtokengate.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ROCM_LIB = "/opt/rocm/lib"
ARCH = "gfx950"

SOURCES = ["k_gate.hip", "k_select.hip", "k_compact.hip", "k_rope.hip", "k_attn.hip", "k_layer.hip", "k_attn_bwd.hip", "k_gate_bwd.hip", "k_gdn.hip", "k_gdn_chunk.hip", "tg_blas.cpp",
           "tg_api.cpp"]

COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-I", INCLUDE, "-I", CSRC, "-Wall",
          "-Wno-unused-function"]
# hipcc -O3 forms packed fp32 ops by itself; they are kept out of the code objects.
DEVICE_ONLY = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *COMMON, "-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".hip"):
        cmd[1:1] = ["-x", "hip"]
        cmd += DEVICE_ONLY
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    noise = "is not a recognized feature for this target"
    msgs = "\n".join(l for l in r.stderr.splitlines() if noise not in l and l.strip())
    if msgs:
        print(f"[{src}]\n{msgs}", file=sys.stderr)
    return obj


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 4)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    # rocBLAS serves the plain GEMMs of the upper-layer projections (tg_linear)
    cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-Wl,--no-undefined", *objs, "-L", ROCM_LIB,
           "-lrocblas", f"-Wl,-rpath,{ROCM_LIB}", "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build()
