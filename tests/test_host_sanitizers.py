"""AddressSanitizer + UndefinedBehaviorSanitizer build of the library's host
code (argument validation, workspace sizing, the codebook and the helpers),
driven through every C ABI path that makes no HIP call.  The GPU code is built
as usual (the sanitizers apply to the host side only: each -fsanitize is
passed behind -Xarch_host)."""

import importlib.util
import os
import shutil
import subprocess
from pathlib import Path

import pytest

ROOT = Path(__file__).resolve().parents[1]
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer", "-g"]


def _build_module():
    spec = importlib.util.spec_from_file_location("_qlora_nf4_build_san", ROOT / "quantized_fine_tuning_amd" / "build.py")
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


@pytest.mark.skipif(shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"),
                    reason="hipcc not available")
def test_host_abi_paths_under_asan_and_ubsan(tmp_path):
    b = _build_module()
    lib = b.build(out=tmp_path / "libqlora_nf4_san.so", extra_flags=SAN)
    exe = tmp_path / "host_abi_driver"
    # the driver is plain C++ against the C header: built by the same LLVM's
    # clang++ in host mode (its sanitizer runtime matches the library's
    # instrumentation)
    clang = Path(b.hipcc()).resolve().parent.parent / "lib" / "llvm" / "bin" / "clang++"
    cmd = [str(clang), "-std=c++17", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-fno-omit-frame-pointer", "-g", "-I", str(ROOT / "include"),
           str(ROOT / "tests" / "sanitize" / "host_abi_driver.cpp"), str(lib), "-o", str(exe),
           f"-Wl,-rpath,{tmp_path}"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stdout + res.stderr
    env = dict(os.environ)
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=0:halt_on_error=1"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    env.pop("LD_PRELOAD", None)
    run = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=300)
    assert run.returncode == 0, run.stdout + run.stderr
    assert "host ABI paths ok" in run.stdout
