"""Build libattn.so for gfx950 with hipcc, in-tree (next to this file).

Usage: ``python -m kv_cache_flashattention_attn_amd.build`` or ``build()``.
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
REPO = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
LIB_NAME = "libattn.so"
LIB_PATH = os.path.join(PKG_DIR, LIB_NAME)
ARCH = "gfx950"


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def command(out: str = LIB_PATH, extra=()) -> list:
    return [
        hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
        # packed fp32 arithmetic stays off: hipcc would otherwise fuse float pairs
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-Wno-unused-result",
        "-I", os.path.join(REPO, "include"), "-I", CSRC,
        *extra,
        os.path.join(CSRC, "attn_lib.hip"), "-o", out,
    ]


def build(verbose: bool = False) -> str:
    """Compile libattn.so (always; never reuses a stale library). Returns its path."""
    tmp = LIB_PATH + ".tmp"
    cmd = command(tmp)
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = [ln for ln in (r.stderr or "").splitlines()
             if "packed-fp32-ops" not in ln or "error" in ln]
    if r.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(noise))
    if verbose and noise:
        print("\n".join(noise), file=sys.stderr)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
