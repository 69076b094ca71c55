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


ASM_PATH = os.path.join(PKG_DIR, "libattn_gfx950.s")  # device assembly, for hazard_scan


def asm_command(out: str = ASM_PATH) -> list:
    """The same device code as the library, as gfx950 assembly text."""
    cmd = command(out)
    cmd.remove("-shared")
    cmd.remove("-fPIC")
    return cmd[:1] + ["--cuda-device-only", "-S"] + cmd[1:]


def build(verbose: bool = False) -> str:
    """Compile libattn.so (always; never reuses a stale library) and, alongside, the
    device assembly that tests/test_build_hazards.py checks. Returns the library path."""
    tmp, tmp_asm = LIB_PATH + ".tmp", ASM_PATH + ".tmp"
    cmd, acmd = command(tmp), asm_command(tmp_asm)
    if verbose:
        print(" ".join(cmd), flush=True)
    procs = [subprocess.Popen(c, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True) for c in (cmd, acmd)]
    results = [(p.wait(), p.communicate()[1]) for p in procs]
    for (rc, err), what in zip(results, ("library", "assembly")):
        noise = [ln for ln in (err or "").splitlines()
                 if ("packed-fp32-ops" not in ln and "hip-link" not in ln) or "error" in ln]
        if rc != 0:
            raise RuntimeError(f"hipcc ({what}) failed:\n" + "\n".join(noise))
        if verbose and noise and what == "library":
            print("\n".join(noise), file=sys.stderr)
    os.replace(tmp, LIB_PATH)
    os.replace(tmp_asm, ASM_PATH)
    return LIB_PATH


ASAN_LIB_PATH = os.path.join(PKG_DIR, "libattn_asan.so")


def build_asan(verbose: bool = False) -> str:
    """A host-AddressSanitizer build of the library (host code only; the device code
    is the ordinary one), for the block pool's and the argument checks' CPU tests:
    tests/run_asan.py loads it with the sanitizer runtime preloaded."""
    cmd = command(ASAN_LIB_PATH + ".tmp", extra=("-g", "-Xarch_host", "-fsanitize=address",
                                                  "-Xarch_host", "-fno-omit-frame-pointer"))
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc (asan) failed:\n" + (r.stderr or ""))
    os.replace(ASAN_LIB_PATH + ".tmp", ASAN_LIB_PATH)
    return ASAN_LIB_PATH


if __name__ == "__main__":
    print(build_asan(verbose=True) if "--asan" in sys.argv else build(verbose=True))
