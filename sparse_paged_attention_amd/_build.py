"""Builds libspa.so (HIP, gfx950) in-tree with hipcc."""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
ROOT = os.path.dirname(PKG)
LIB = os.path.join(PKG, "libspa.so")
SOURCES = ["api.cpp", "pool.hip", "select.hip", "attn.hip", "prefill.hip", "probe.hip"]
ARCH = "gfx950"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# Packed fp32 instructions are kept out of every kernel.
FLAGS = ["-O3", "-std=c++17", "-fPIC", "-Wall", f"--offload-arch={ARCH}",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         f"-I{os.path.join(ROOT, 'include')}"]


class BuildError(RuntimeError):
    pass


def _run(cmd: list) -> None:
    """Runs one compiler command. Its output (the compiler's diagnostics) is
    printed when the command fails, or always with SPA_BUILD_VERBOSE set;
    hipcc's host pass warning about the packed-fp32 target feature is the only
    expected output of a good build."""
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if res.returncode != 0 or os.environ.get("SPA_BUILD_VERBOSE"):
        sys.stderr.write(res.stdout)
    if res.returncode != 0:
        raise BuildError(f"command failed with exit status {res.returncode}: {' '.join(cmd)}\n"
                         f"{res.stdout[-4000:]}")


def _compile(src: str, out_dir: str) -> str:
    obj = os.path.join(out_dir, src + ".o")
    lang = ["-x", "hip"] if src.endswith(".hip") else []
    _run([HIPCC, *FLAGS, *lang, "-c", os.path.join(CSRC, src), "-o", obj])
    return obj


def build_library() -> str:
    out_dir = os.path.join(PKG, "_build")
    os.makedirs(out_dir, exist_ok=True)
    with ThreadPoolExecutor(len(SOURCES)) as ex:
        objs = list(ex.map(lambda s: _compile(s, out_dir), SOURCES))
    tmp = LIB + ".tmp"
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs])
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build_library())
