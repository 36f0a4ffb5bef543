"""HIP test programs (not part of the product library), built in-tree with
hipcc for gfx950 next to their sources."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
PROGRAMS = ["quantizer_check"]


def path(name: str) -> str:
    return os.path.join(HERE, name)


def build(force: bool = False) -> None:
    for name in PROGRAMS:
        out = path(name)
        if os.path.exists(out) and not force:
            continue
        cmd = [HIPCC, "-O3", "-std=c++17", "--offload-arch=gfx950",
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
               f"-I{os.path.join(ROOT, 'include')}",
               f"-I{os.path.join(ROOT, 'sparse_paged_attention_amd', 'csrc')}",
               path(name + ".hip"), "-o", out + ".tmp"]
        res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
        if res.returncode != 0:
            raise RuntimeError(f"building {name} failed:\n{res.stdout[-4000:]}")
        os.replace(out + ".tmp", out)
