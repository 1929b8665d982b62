"""Build libw4a16.so (hand-written HIP for gfx950) and the benchmark's HBM
calibration library libw4a16_calib.so in-tree with hipcc.

Usage: python -m block_scaled_fp4_w4a16_amd.build
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SRC = os.path.join(PKG, "csrc", "w4a16.hip")
LIB = os.path.join(PKG, "libw4a16.so")
CALIB_SRC = os.path.join(PKG, "csrc", "calib.hip")
CALIB_LIB = os.path.join(PKG, "libw4a16_calib.so")
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libw4a16.so)")


def build_command(out: str, extra=(), src: str = SRC) -> list:
    return [
        hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-shared", "-fPIC",
        # no packed-fp32 VALU instructions (v_pk_fma_f32 and friends)
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        # one-lane atomics stay plain: the optimizer's lane combining would wait
        # for the batch counter's result right after issuing it
        "-mllvm", "-amdgpu-atomic-optimizer-strategy=None",
        "-I", os.path.join(ROOT, "include"), "-I", os.path.join(PKG, "csrc"),
        *extra, "-o", out, src,
    ]


def build(extra=(), out: str = LIB, verbose: bool = False, src: str = SRC) -> str:
    tmp = out + ".tmp"
    cmd = build_command(tmp, extra, src)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed ({res.returncode}) building {out}")
    if verbose:
        err = "\n".join(l for l in res.stderr.splitlines() if "packed-fp32-ops" not in l)
        if err.strip():
            sys.stderr.write(err + "\n")
    os.replace(tmp, out)
    return out


def build_calib(verbose: bool = False) -> str:
    """The benchmark's HBM read calibration kernel (not part of the matmul ABI)."""
    return build(out=CALIB_LIB, verbose=verbose, src=CALIB_SRC)


if __name__ == "__main__":
    print(build(verbose=True))
    print(build_calib(verbose=True))
