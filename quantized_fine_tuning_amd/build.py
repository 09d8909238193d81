"""Builds libqlora_nf4.so (HIP, gfx950) in-tree with hipcc.

    python -m quantized_fine_tuning_amd.build

Flags: -O3; no fast-math; fp contraction off (every fp32 operation rounds once,
which the bit-exact parts of the library rely on); correctly rounded fp32
division and square root; packed-fp32 instruction selection disabled.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys
from pathlib import Path

PKG = Path(__file__).resolve().parent
CSRC = PKG / "csrc"
LIB = PKG / "libqlora_nf4.so"
SOURCES = ["codebook.cpp", "capi.cpp", "quantize.hip", "gemm.hip", "fwd.hip", "dx.hip", "gemv.hip"]
ARCH = "gfx950"

FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "-shared",
    f"--offload-arch={ARCH}",
    "-ffp-contract=off",
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-fno-gpu-rdc",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unused-command-line-argument",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and Path(cand).exists():
            return cand
    raise RuntimeError("hipcc not found")


def build(verbose: bool = False) -> Path:
    tmp = LIB.with_suffix(".so.tmp")
    cmd = [hipcc(), *FLAGS, "-I", str(CSRC), "-o", str(tmp)]
    for s in SOURCES:
        src = CSRC / s
        if src.suffix == ".cpp":
            cmd += ["-x", "hip", str(src)]
        else:
            cmd += ["-x", "hip", str(src)]
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
