"""The C-ABI host layer (hs2_api.cpp) built for the CPU with AddressSanitizer and
UndefinedBehaviorSanitizer, its kernel launchers replaced by host-only stand-ins
(tests/host/launch_stubs.cpp), running the boundary tests and every launch sequence in
a child process.  Any sanitizer report fails the child (UBSan aborts on the first
finding; ASan on its first error).  CPU only: nothing here touches a GPU."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "long_context_decode_full_amd", "csrc")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def _runtime(name):
    out = subprocess.run(["g++", f"-print-file-name={name}"], capture_output=True, text=True).stdout.strip()
    return out if os.path.isabs(out) and os.path.exists(out) else None


@pytest.fixture(scope="module")
def host_build(tmp_path_factory):
    if shutil.which("g++") is None or not os.path.exists(os.path.join(ROCM, "include", "hip")):
        pytest.skip("needs g++ and the ROCm headers")
    asan, ubsan = _runtime("libasan.so"), _runtime("libubsan.so")
    if asan is None or ubsan is None:
        pytest.skip("sanitizer runtimes not installed")
    out = str(tmp_path_factory.mktemp("host_asan") / "libhs2_host.so")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fPIC", "-shared", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
           "-D__HIP_PLATFORM_AMD__", '-DHS2_BUILD_ID="host-sanitizer-build"',
           "-I", os.path.join(ROCM, "include"), "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           os.path.join(CSRC, "hs2_api.cpp"), os.path.join(ROOT, "tests", "host", "launch_stubs.cpp"),
           "-L", os.path.join(ROCM, "lib"), "-lamdhip64", f"-Wl,-rpath,{os.path.join(ROCM, 'lib')}", "-o", out]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stdout + res.stderr
    return out, asan, ubsan


def test_host_layer_under_asan_and_ubsan(host_build):
    lib, asan, ubsan = host_build
    env = dict(os.environ, HS2_HOST_LIB=lib, LD_PRELOAD=f"{asan}:{ubsan}",
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    cmd = [sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
           os.path.join(ROOT, "tests", "test_boundary.py"),
           os.path.join(ROOT, "tests", "test_host_launch_paths.py")]
    res = subprocess.run(cmd, capture_output=True, text=True, env=env, cwd=ROOT, timeout=600)
    tail = (res.stdout + res.stderr)[-4000:]
    assert res.returncode == 0, tail
    assert "passed" in res.stdout and "skipped" not in res.stdout.splitlines()[-1], tail
    assert "runtime error" not in res.stderr and "AddressSanitizer" not in res.stderr, tail
