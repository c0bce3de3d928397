"""Builds libpagedattn.so for gfx950 with hipcc, in the package directory.

Usage: python -m exact_tiled_attention_pa_amd.build
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libpagedattn.so")
SOURCES = ["api.cpp", "block_manager.cpp", "prefill.hip", "prefill_split.hip", "decode.hip",
           "decode_gqa.hip", "kv_cache.hip", "decode_static.hip"]

HIP_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    # no packed-fp32 VALU instructions in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def hipcc_path() -> str:
    return os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def build(verbose: bool = False, extra_flags=None) -> str:
    """Compiles every HIP source into libpagedattn.so (always rebuilds)."""
    tmp = LIB + ".tmp"
    cmd = [hipcc_path()] + HIP_FLAGS + list(extra_flags or []) + [
        "-I", INCLUDE, "-I", CSRC] + [os.path.join(CSRC, s) for s in SOURCES] + ["-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed with status {res.returncode}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
