"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer,
on the CPU.

csrc/api.cpp (argument checking, weight layout arithmetic, descriptor checks,
the per-device scratch and arch caches) is built with g++ -fsanitize=address,
undefined together with tests/asan/hip_stubs.cpp, which stands in for the
HIP runtime and the kernel launchers. Then:
  * every check of tests/test_abi.py runs against that build with no device;
  * tests/asan/device_checks.py drives it as if a gfx950 were present (valid
    calls reach exactly one launcher, invalid ones none) and as if another GPU
    were (every launching call is QGEMM_E_DEVICE).
Any sanitizer report aborts the run and fails the test.
"""
import os
import shutil
import subprocess
import sys

import pytest

from conftest import ROOT

GXX = shutil.which("g++")
CSRC = os.path.join(ROOT, "block_scaled_quantized_qgemm_amd", "csrc")
ASAN_DIR = os.path.join(ROOT, "tests", "asan")
HIP_INCLUDE = "/opt/rocm/include"


@pytest.fixture(scope="module")
def asan_lib(tmp_path_factory):
    if not GXX or not os.path.isdir(HIP_INCLUDE):
        pytest.skip("needs g++ and the HIP headers")
    out = str(tmp_path_factory.mktemp("asan") / "libqgemm_asan.so")
    cmd = [GXX, "-std=c++17", "-shared", "-fPIC", "-D__HIP_PLATFORM_AMD__", "-I", HIP_INCLUDE, "-I", CSRC,
           "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer",
           "-g", "-O1", os.path.join(CSRC, "api.cpp"), os.path.join(ASAN_DIR, "hip_stubs.cpp"), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-4000:]
    return out


def _run(args, mode):
    libasan = subprocess.run([GXX, "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    env = dict(os.environ, LD_PRELOAD=libasan, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1", QGEMM_STUB_DEVICE=mode)
    r = subprocess.run([sys.executable] + args, capture_output=True, text=True, env=env, timeout=600)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-6000:]
    assert r.returncode == 0, out[-6000:]
    return out


def test_abi_checks_under_sanitizers(asan_lib):
    out = _run([os.path.join(ASAN_DIR, "run_abi_tests.py"), asan_lib], "none")
    assert " passed" in out


def test_device_paths_under_sanitizers(asan_lib, tmp_path):
    descs = str(tmp_path / "descs.bin")
    for mode in ("gfx950", "gfx942"):
        out = _run([os.path.join(ASAN_DIR, "device_checks.py"), asan_lib, mode, descs], mode)
        assert f"device checks passed ({mode})" in out
