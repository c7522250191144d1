"""Build step of the HIP library: hipcc for gfx950, in-tree.

Compiles every source under ``csrc/`` to an object in ``<repo>/_build/`` and
links ``libglahybrid.so`` next to this file.  Run ``python -m
gated_linear_attention_hybrid_amd.build_lib`` (or ``__graft_entry__.build()``).
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
LIB = os.path.join(PKG, "libglahybrid.so")
ARCH = "gfx950"

SOURCES = ["capi.cpp", "recurrent.hip", "chunked.hip", "chunk_out.hip", "decode.hip", "backward.hip", "delta.hip", "serving.hip", "swa_wide.hip", "delta_chunk.hip", "bwd_window.hip",
           "bwd_walk.hip", "bwd_feat.hip",
           "bwd_prep.hip"]

# -packed-fp32-ops: keep the compiler from emitting packed fp32 VALU
# instructions (ordinary float code is used everywhere instead).
COMMON = ["-O3", "-std=c++17", "-fPIC", "--offload-arch=" + ARCH,
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-I" + INCLUDE, "-I" + CSRC, "-Wall", "-Wno-unused-function"]

# Per-source extras.  delta_chunk.hip: matrix-core results in ordinary VGPRs
# (its recurrence feeds most of them to vector instructions, and results in
# the accumulator registers would need a copy each).
EXTRA = {"delta_chunk.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]}


def _hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", "hipcc"):
        if cand and (os.path.sep not in cand or os.path.exists(cand)):
            return cand
    raise RuntimeError("hipcc not found")


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [_hipcc()] + COMMON + EXTRA.get(src, []) + ["-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".cpp"):
        cmd[1:1] = ["-x", "hip"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s%s" % (src, r.stdout, r.stderr))
    return obj


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [_hipcc(), "-shared", "-fPIC", "--offload-arch=" + ARCH] + objs + ["-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n%s%s" % (r.stdout, r.stderr))
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    build()
    sys.exit(0)
