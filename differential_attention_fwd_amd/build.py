"""Build libdiffattn.so (HIP for gfx950) in-tree with hipcc.

Every HIP source is compiled with packed-FP32 instructions disabled (-Xclang -target-feature -Xclang
-packed-fp32-ops); hipcc's host pass warns that it does not know that feature, which is harmless.
"""
from __future__ import annotations

import concurrent.futures
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libdiffattn.so")
SOURCES = ["diffattn_api.cpp", "prefill_bf16.hip", "decode_bf16.hip", "attn_f32.hip", "backward_bf16.hip"]
# Per-source extra flags.  The prefill kernel never produces a NaN (see its header), and without NaN semantics
# v_max3 needs no quieting of MFMA results.
EXTRA = {"prefill_bf16.hip": ["-fno-honor-nans"]}
HEADERS = ["launch.h", "tiles.h"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = ["-x", "hip", f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I", os.path.join(ROOT, "include")]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, *EXTRA.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    msg = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{msg}")
    if msg.strip():
        sys.stderr.write(msg + "\n")
    return obj


def build(verbose: bool = False) -> str:
    """Compile every HIP source for gfx950 and link libdiffattn.so next to this file.  Always rebuilds."""
    os.makedirs(BUILD, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
