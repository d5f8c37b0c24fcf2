"""Build the HIP library ``libjetlong.so`` in-tree for gfx950 with hipcc.

``python -m zero_shot_rope_attention_amd.build`` (or ``build()``) compiles every
source under ``csrc/`` into ``zero_shot_rope_attention_amd/libjetlong.so``.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_NAME = "libjetlong.so"
LIB_PATH = os.path.join(PKG_DIR, LIB_NAME)
SOURCES = ["jl_api.cpp", "jl_prefill.hip", "jl_decode.hip", "jl_layer.hip"]
ARCH = "gfx950"

# Packed-fp32 VALU forms are disabled for all device code; plain fp32 is used instead.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


# rocBLAS serves the projections of the attention layer (plain library GEMMs).
LINK_FLAGS = ["-L/opt/rocm/lib", "-Wl,-rpath,/opt/rocm/lib", "-lrocblas"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def build(verbose: bool = False) -> str:
    """Compile the library (always, even if an older build exists); returns its path."""
    tmp = LIB_PATH + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
           "-Wall", "-Wno-unused-function", "-I", INCLUDE, "-I", CSRC, *DEVICE_FLAGS,
           "-o", tmp] + [os.path.join(CSRC, s) for s in SOURCES] + LINK_FLAGS
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{res.stdout}\n{res.stderr}")
    if verbose and res.stderr.strip():
        print(res.stderr, file=sys.stderr)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
