"""Build the HIP library ``libjetlong.so`` in-tree for gfx950 with hipcc.

``python -m zero_shot_rope_attention_amd.build`` (or ``build()``) compiles every
source under ``csrc/`` into ``zero_shot_rope_attention_amd/libjetlong.so``.

``python -m zero_shot_rope_attention_amd.build --sanitize`` (``build(sanitize=True)``)
builds ``libjetlong_asan.so`` instead: the same sources with the host code
instrumented by AddressSanitizer and UndefinedBehaviorSanitizer (argument
checks, workspace sizing, launch planning); device code is built as usual.  The
binding loads it when ``JL_LIBRARY`` names it; the process must preload the ASan
runtime (``asan_runtime()``), e.g.::

    LD_PRELOAD=$(python -c 'from zero_shot_rope_attention_amd.build import asan_runtime; print(asan_runtime())') \
    ASAN_OPTIONS=detect_leaks=0 JL_LIBRARY=zero_shot_rope_attention_amd/libjetlong_asan.so \
    python -m pytest tests/test_abi_cpu.py
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
ASAN_LIB_PATH = os.path.join(PKG_DIR, "libjetlong_asan.so")
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


# Host-only sanitizers: each -fsanitize= applies to the host compilation alone.
SANITIZE_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                  "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer",
                  "-shared-libsan", "-g"]


def asan_runtime() -> str:
    """Path of the clang ASan runtime the sanitized library needs preloaded."""
    import glob
    cands = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not cands:
        raise RuntimeError("clang ASan runtime not found")
    return cands[-1]


def build(verbose: bool = False, sanitize: bool = False) -> str:
    """Compile the library (always, even if an older build exists); returns its path."""
    out = ASAN_LIB_PATH if sanitize else LIB_PATH
    tmp = out + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-O1" if sanitize else "-O3", "-std=c++17", "-fPIC", "-shared",
           "-Wall", "-Wno-unused-function", "-I", INCLUDE, "-I", CSRC, *DEVICE_FLAGS,
           *(SANITIZE_FLAGS if sanitize else []),
           "-o", tmp] + [os.path.join(CSRC, s) for s in SOURCES] + LINK_FLAGS
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{res.stdout}\n{res.stderr}")
    if verbose and res.stderr.strip():
        print(res.stderr, file=sys.stderr)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True, sanitize="--sanitize" in sys.argv[1:]))
