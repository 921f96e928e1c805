"""Build libpkv.so (the HIP kernels and the C ABI) for gfx950 with hipcc.

Usage: ``python -m paged_kv_cache_317_amd.build`` or ``build()`` from Python.
The library lands next to this file; the Python binding loads it from there.
"""

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_PATH = os.path.join(HERE, "libpkv.so")
ARCH = "gfx950"

SOURCES = ["attn_decode.hip", "attn_extend.hip", "kv_write.hip", "block_copy.hip",
           "decode_noalloc.hip", "pkv_api.cpp", "block_manager.cpp"]

# Packed fp32 instructions are kept out of the generated code on purpose.
HIP_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-fvisibility=hidden", "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def hipcc_path():
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found; set HIPCC or install ROCm")


def build(out=LIB_PATH, extra_flags=(), verbose=False):
    """Compile every source into ``out``; returns its path."""
    tmp = out + ".tmp"
    cmd = [hipcc_path(), *HIP_FLAGS, *extra_flags, "-I", INCLUDE,
           *[os.path.join(CSRC, s) for s in SOURCES], "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{res.stderr}")
    if verbose and res.stderr.strip():
        print(res.stderr, file=sys.stderr)
    os.replace(tmp, out)
    return out


def ensure_built():
    """Build only when no library is present (tests, smoke and bench use this)."""
    if not os.path.exists(LIB_PATH):
        build()
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
