"""Builds libqlora_nf4.so (HIP, gfx950) in-tree with hipcc.

    python quantized_fine_tuning_amd/build.py

(run as a file: importing the package first would load the library it builds)

Flags: -O3; no fast-math; fp contraction off (every fp32 operation rounds once,
which the bit-exact parts of the library rely on); correctly rounded fp32
division and square root; packed-fp32 instruction selection disabled.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor
from pathlib import Path

PKG = Path(__file__).resolve().parent
CSRC = PKG / "csrc"
INCLUDE = PKG.parent / "include"  # the C ABI header
LIB = PKG / "libqlora_nf4.so"
SOURCES = ["codebook.cpp", "capi.cpp", "quantize.hip", "linear.hip", "lora.hip", "fwd.hip", "dx.hip", "gemv.hip", "adamw.hip", "merge.hip", "variants.hip", "peak.hip", "splitk.hip"]
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


def build(verbose: bool = False, csrc: Path = CSRC, out: Path = LIB, extra_flags=()) -> Path:
    """Compiles every source to an object (in parallel), then links.
    extra_flags go on every compile and the link line (a sanitizer build of
    the host code passes ``-Xarch_host -fsanitize=...`` here)."""
    objdir = out.parent / "_build"
    objdir.mkdir(exist_ok=True)
    cc = hipcc()

    def compile_one(name: str) -> Path:
        obj = objdir / (name + ".o")
        cmd = [cc, *[f for f in FLAGS if f != "-shared"], *extra_flags, "-c", "-I", str(csrc), "-I", str(INCLUDE), "-x", "hip",
               str(csrc / name), "-o", str(obj)]
        if verbose:
            print(" ".join(cmd), flush=True)
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            sys.stderr.write(res.stdout + res.stderr)
            raise RuntimeError(f"hipcc failed on {name} with status {res.returncode}")
        return obj

    jobs = min(len(SOURCES), max(1, int(os.environ.get("MAX_JOBS", os.cpu_count() or 1))))
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    tmp = out.with_suffix(".so.tmp")
    cmd = [cc, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-fno-gpu-rdc", *extra_flags, "-o", str(tmp),
           *map(str, objs)]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"link failed with status {res.returncode}")
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
