"""Ahead-of-time build of libpsa_attn.so for gfx950 with hipcc.

The library is built in-tree, next to this file, so that it travels with the
source tree; nothing is JIT-compiled at import time.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_NAME = "libpsa_attn.so"
LIB_PATH = os.path.join(PKG_DIR, LIB_NAME)
OFFLOAD_ARCH = "gfx950"

# Packed-fp32 VALU forms are disabled for all device code.
COMMON_DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                       # non-IEEE mode: max/min need no NaN canonicalisation (device code
                       # only; the host-side argument checks still see real NaNs)
                       "-Xarch_device", "-mno-amdgpu-ieee", "-Xarch_device", "-fno-honor-nans",
                       # kernel arguments preloaded into SGPRs at dispatch instead of
                       # loaded by the first instructions (the code keeps a prologue for
                       # firmware without it); measured 2-3 % on the short forward calls
                       "-mllvm", "-amdgpu-kernarg-preload-count=16"]
# The attention kernels keep MFMA accumulators in ordinary VGPRs: the softmax
# reads and rescales them with VALU ops, which cannot address AGPRs.
VGPR_ACC_FLAGS = ["-mllvm", "-amdgpu-mfma-vgpr-form"]
DEVICE_FLAGS = COMMON_DEVICE_FLAGS + VGPR_ACC_FLAGS


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (set HIPCC or install ROCm)")


def sources() -> list[tuple[str, list[str]]]:
    """(source, device flags) of each translation unit: the attention kernels
    and the C ABI with VGPR accumulators; the wide-tile convolution GEMM with
    its accumulators in AGPRs."""
    return [(os.path.join(CSRC, "psa_attn.hip"), DEVICE_FLAGS),
            (os.path.join(CSRC, "psa_conv_wide.hip"), COMMON_DEVICE_FLAGS)]


def _run(cmd: list[str], verbose: bool) -> subprocess.Popen:
    if verbose:
        print(" ".join(cmd), flush=True)
    return subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)


def _finish(proc: subprocess.Popen, verbose: bool) -> None:
    out, _ = proc.communicate()
    # hipcc's host pass does not know the device-only feature flag; that
    # warning is expected and harmless, everything else is shown.
    noise = "is not a recognized feature for this target"
    msgs = [ln for ln in out.splitlines() if noise not in ln]
    if proc.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs), file=sys.stderr)


def build_library(verbose: bool = False, extra: list[str] | None = None, out: str | None = None) -> str:
    """Compile the HIP kernels and the C ABI into libpsa_attn.so (always
    recompiles): each translation unit to an object (in parallel), then one
    shared library.  `extra` appends compiler flags and `out` redirects the
    output path.  Returns the library path."""
    target = out or LIB_PATH
    tmp = target + ".tmp"
    base = [hipcc(), f"--offload-arch={OFFLOAD_ARCH}", "-O3", "-std=c++17", "-fPIC",
            "-Wall", "-Wno-unused-command-line-argument", f"-I{INCLUDE}", f"-I{CSRC}"]
    with tempfile.TemporaryDirectory(prefix="psa_build_") as tmpdir:
        objs, procs = [], []
        for src, flags in sources():
            obj = os.path.join(tmpdir, os.path.basename(src) + ".o")
            objs.append(obj)
            procs.append(_run([*base, *flags, "-c", src, "-o", obj, *(extra or [])], verbose))
        for p in procs:
            _finish(p, verbose)
        _finish(_run([hipcc(), f"--offload-arch={OFFLOAD_ARCH}", "-fPIC", "-shared", *objs, "-o", tmp], verbose),
                verbose)
    os.replace(tmp, target)
    return target


if __name__ == "__main__":
    print(build_library(verbose=True))
