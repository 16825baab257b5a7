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
CHECK_BUILD = os.path.join(BUILD, "check")
CHECK_LIB = os.path.join(HERE, "libdiffattn_check.so")
# Measurement context for bench.py (a streaming-read probe), not part of the library.
PROBE_SRC = "stream_probe.hip"
PROBE_LIB = os.path.join(HERE, "libstreamprobe.so")
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


def _compile(src: str, check: bool = False) -> str:
    obj = os.path.join(CHECK_BUILD if check else BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, *EXTRA.get(src, []), *(["-DDIFFATTN_CHECK"] if check else []), "-c",
           os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    msg = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{msg}")
    if msg.strip():
        sys.stderr.write(msg + "\n")
    return obj


def _link(objs, lib):
    tmp = lib + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}{r.stderr}")
    os.replace(tmp, lib)


def build(verbose: bool = False) -> str:
    """Compile every HIP source for gfx950 and link libdiffattn.so next to this file, and the check build
    libdiffattn_check.so (-DDIFFATTN_CHECK: every LDS piece is filled with NaN before its direct load is issued, so a
    read that races ahead of a load shows up as NaN in the output; for tests only).  Always rebuilds."""
    os.makedirs(BUILD, exist_ok=True)
    os.makedirs(CHECK_BUILD, exist_ok=True)
    jobs = [(s, False) for s in SOURCES] + [(s, True) for s in SOURCES] + [(PROBE_SRC, False)]
    with concurrent.futures.ThreadPoolExecutor(max_workers=len(jobs)) as ex:
        objs = list(ex.map(lambda j: _compile(*j), jobs))
    n = len(SOURCES)
    _link(objs[:n], LIB)
    _link(objs[n:2 * n], CHECK_LIB)
    _link(objs[2 * n:], PROBE_LIB)
    if verbose:
        print(f"built {LIB}, {CHECK_LIB} and {PROBE_LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
