"""The C-ABI validation layer under AddressSanitizer and UndefinedBehavior-
Sanitizer, on the CPU.  fa_api.cpp is compiled for the host alone with g++
and linked with launchers that only report failure (tests/abi_launch_stubs.cpp),
so no GPU code is built or run; the ABI tests (tests/test_abi.py) then run
against that library in a fresh process with the sanitizer runtime loaded
first.  Any sanitizer report fails the test."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ROCM_INCLUDE = "/opt/rocm/include"


def _asan_runtime():
    gxx = shutil.which("g++")
    if gxx is None:
        return None
    path = subprocess.run([gxx, "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


@pytest.mark.skipif(_asan_runtime() is None or not os.path.isdir(ROCM_INCLUDE),
                    reason="needs g++ with libasan and the ROCm headers")
def test_validation_layer_clean_under_sanitizers(tmp_path):
    lib = tmp_path / "libmiattn_hostcheck.so"
    srcs = [os.path.join(ROOT, "tiled_attention_fa_amd", "csrc", "fa_api.cpp"),
            os.path.join(ROOT, "tests", "abi_launch_stubs.cpp")]
    build = subprocess.run(
        ["g++", "-std=c++17", "-O1", "-g", "-fPIC", "-shared", "-fno-omit-frame-pointer",
         "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-D__HIP_PLATFORM_AMD__",
         f"-I{ROCM_INCLUDE}", *srcs, "-o", str(lib)], capture_output=True, text=True)
    assert build.returncode == 0, build.stderr
    env = dict(os.environ, MIATTN_ABI_TEST_LIB=str(lib), LD_PRELOAD=_asan_runtime(),
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    run = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", "-m", "not gpu",
                          os.path.join(ROOT, "tests", "test_abi.py")],
                         capture_output=True, text=True, env=env, cwd=ROOT, timeout=600)
    out = run.stdout + run.stderr
    assert run.returncode == 0, out[-4000:]
    for marker in ("ERROR: AddressSanitizer", "runtime error:", "ERROR: LeakSanitizer"):
        assert marker not in out, out[-4000:]
    assert " passed" in run.stdout, out[-2000:]
