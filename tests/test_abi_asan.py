"""The host side of the C ABI under AddressSanitizer: api.cpp (argument
checks, launch planning, workspace sizing, the page allocator) is built by g++
with -fsanitize=address together with host-only stand-ins for the kernel
launchers (tests/asan/launch_stubs.cpp), and the ABI tests run against that
build in a child process with the sanitizer's runtime preloaded. Any heap or
stack error in the host code fails the child. CPU only: no GPU code is built
or run here."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _libasan() -> str:
    p = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    if not p or not os.path.exists(p):
        pytest.skip("gcc's libasan.so not found")
    return p


def test_abi_checks_under_address_sanitizer(tmp_path):
    asan = _libasan()
    lib = str(tmp_path / "libspa_asan.so")
    flags = ["-std=c++17", "-O1", "-g", "-fPIC", "-fsanitize=address", "-fno-omit-frame-pointer",
             "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", f"-I{os.path.join(ROOT, 'include')}"]
    srcs = [os.path.join(ROOT, "sparse_paged_attention_amd", "csrc", "api.cpp"),
            os.path.join(ROOT, "tests", "asan", "launch_stubs.cpp")]
    build = subprocess.run(["g++", *flags, "-shared", "-o", lib, *srcs], capture_output=True, text=True)
    assert build.returncode == 0, build.stderr[-4000:]
    env = dict(os.environ, SPA_LIB_PATH=lib, LD_PRELOAD=asan,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=0:halt_on_error=1:exitcode=86")
    res = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                          os.path.join(ROOT, "tests", "test_abi.py")],
                         cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    tail = (res.stdout + res.stderr)[-6000:]
    assert "ERROR: AddressSanitizer" not in tail, tail
    assert res.returncode == 0, tail
    assert " passed" in res.stdout and "skipped" not in res.stdout.split("\n")[-2], tail
