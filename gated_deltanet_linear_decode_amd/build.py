"""Compile the HIP library (libgdn_block.so) in-tree for gfx950.

    python -m gated_deltanet_linear_decode_amd.build           # libgdn_block.so
    python -m gated_deltanet_linear_decode_amd.build --trace   # libgdn_block_trace.so: the same
        kernels with per-workgroup wall-clock stamps (GDN_TRACE), read by
        python -m gated_deltanet_linear_decode_amd.timeline
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
LIB = os.path.join(PKG, "libgdn_block.so")
TRACE_LIB = os.path.join(PKG, "libgdn_block_trace.so")
SOURCES = [os.path.join(PKG, "csrc", "gdn_block.hip")]
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-shared", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def build(verbose: bool = False, trace: bool = False) -> str:
    """Compile every source into the shared library (with `trace`, the profiling build);
    returns its path."""
    lib = TRACE_LIB if trace else LIB
    tmp = lib + ".tmp"
    cmd = [HIPCC, *FLAGS, *(["-DGDN_TRACE"] if trace else []), "-I", os.path.join(ROOT, "include"), *SOURCES,
           "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    errs = [ln for ln in res.stderr.splitlines() if "packed-fp32-ops" not in ln]
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(errs))
    if verbose and errs:
        print("\n".join(errs), file=sys.stderr)
    os.replace(tmp, lib)
    return lib


if __name__ == "__main__":
    print(build(verbose=True, trace="--trace" in sys.argv[1:]))
