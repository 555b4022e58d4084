"""The C ABI layer under AddressSanitizer and UndefinedBehaviorSanitizer.

fa_api.cpp (argument validation, workspace sizing, dispatch) is built with
g++ for the host only, linked with host stubs of the kernel launchers
(tests/asan/fa_launch_stubs.cpp), and the ABI tests of tests/test_abi.py run
against that build in a child process with the sanitizer runtime preloaded.
No GPU code is built or run here.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OUT_DIR = os.path.join(ROOT, "_build", "asan")
LIB = os.path.join(OUT_DIR, "libflash_attn_abi_asan.so")


def _runtime(name: str) -> str | None:
    gxx = shutil.which("g++")
    if gxx is None:
        return None
    path = subprocess.run([gxx, f"-print-file-name={name}"], capture_output=True, text=True).stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


@pytest.fixture(scope="module")
def asan_lib():
    gxx = shutil.which("g++")
    asan = _runtime("libasan.so")
    if gxx is None or asan is None or not os.path.isdir("/opt/rocm/include"):
        pytest.skip("g++ with libasan and the ROCm headers are needed")
    os.makedirs(OUT_DIR, exist_ok=True)
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
           "-shared", "-fPIC", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
           "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROOT, "exact_io_aware_47_amd", "csrc"),
           os.path.join(ROOT, "exact_io_aware_47_amd", "csrc", "fa_api.cpp"),
           os.path.join(ROOT, "tests", "asan", "fa_launch_stubs.cpp"),
           "-o", LIB]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, f"sanitizer build failed:\n{' '.join(cmd)}\n{res.stderr}"
    return asan


def test_abi_layer_clean_under_sanitizers(asan_lib):
    env = dict(os.environ)
    env["LD_PRELOAD"] = asan_lib
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1:abort_on_error=0"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    env["FA_ABI_STUB_LIB"] = LIB
    env["CUDA_VISIBLE_DEVICES"] = ""
    env["HIP_VISIBLE_DEVICES"] = ""
    res = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                          os.path.join(ROOT, "tests", "test_abi.py"), "-m", "not gpu"],
                         capture_output=True, text=True, env=env, cwd=ROOT, timeout=600)
    out = res.stdout + res.stderr
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert res.returncode == 0, out[-4000:]
    assert " passed" in res.stdout and "skipped" not in res.stdout.split("\n")[-2], res.stdout[-2000:]
