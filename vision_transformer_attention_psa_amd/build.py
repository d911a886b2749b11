"""Ahead-of-time build of libpsa_attn.so for gfx950 with hipcc.

The library is built in-tree, next to this file, so that it travels with the
source tree; nothing is JIT-compiled at import time.
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
LIB_NAME = "libpsa_attn.so"
LIB_PATH = os.path.join(PKG_DIR, LIB_NAME)
OFFLOAD_ARCH = "gfx950"

# Packed-fp32 VALU forms are disabled for all device code.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                # keep MFMA accumulators in ordinary VGPRs: the softmax reads and
                # rescales them with VALU ops, which cannot address AGPRs
                "-mllvm", "-amdgpu-mfma-vgpr-form",
                # non-IEEE mode: max/min need no NaN canonicalisation (device code
                # only; the host-side argument checks still see real NaNs)
                "-Xarch_device", "-mno-amdgpu-ieee", "-Xarch_device", "-fno-honor-nans"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (set HIPCC or install ROCm)")


def sources() -> list[str]:
    return [os.path.join(CSRC, "psa_attn.hip")]


def build_library(verbose: bool = False, extra: list[str] | None = None, out: str | None = None) -> str:
    """Compile the HIP kernels and the C ABI into libpsa_attn.so (always
    recompiles).  `extra` appends compiler flags (e.g. tile overrides) and
    `out` redirects the output path.  Returns the library path."""
    target = out or LIB_PATH
    tmp = target + ".tmp"
    cmd = [hipcc(), f"--offload-arch={OFFLOAD_ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
           "-Wall", "-Wno-unused-command-line-argument", *DEVICE_FLAGS,
           f"-I{INCLUDE}", f"-I{CSRC}", *sources(), "-o", tmp, *(extra or [])]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the device-only feature flag; that
    # warning is expected and harmless, everything else is shown.
    noise = "is not a recognized feature for this target"
    msgs = [ln for ln in (res.stdout + res.stderr).splitlines() if noise not in ln]
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs), file=sys.stderr)
    os.replace(tmp, target)
    return target


if __name__ == "__main__":
    print(build_library(verbose=True))
