"""Build libbonsai.so (the gfx950 kernels and the C ABI) in-tree: hipcc for the kernel sources
(*.hip), the host compiler for the host-only part of the C ABI (*.cpp)."""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor
from pathlib import Path

PKG = Path(__file__).resolve().parent
ROOT = PKG.parent
CSRC = PKG / "csrc"
OUT = PKG / "_lib" / "libbonsai.so"
OBJ = ROOT / "_build" / "obj"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CXX = os.environ.get("CXX", "g++")
HOST_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-Wall", "-Wextra", f"-I{ROOT / 'include'}"]
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # packed fp32 VALU forms are kept out of every kernel
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # the kernel arguments arrive preloaded in SGPRs, so a wave's first instructions do not wait
    # on a scalar load of the argument block (about 0.2 us of a 4-6 us decode call)
    "-mllvm", "-amdgpu-kernarg-preload-count=16",
    f"-I{ROOT / 'include'}",
]


def sources() -> list[Path]:
    return sorted(CSRC.glob("*.hip")) + sorted(CSRC.glob("*.cpp"))


def build(verbose: bool = False) -> Path:
    """Compile every kernel source for gfx950 and link the shared library (always rebuilds)."""
    OBJ.mkdir(parents=True, exist_ok=True)
    OUT.parent.mkdir(parents=True, exist_ok=True)

    def compile_one(src: Path) -> Path:
        obj = OBJ / (src.stem + ".o")
        if src.suffix == ".cpp":
            cmd = [CXX, *HOST_FLAGS, "-c", str(src), "-o", str(obj)]
        else:
            cmd = [HIPCC, *FLAGS, "-c", str(src), "-o", str(obj)]
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            sys.stderr.write(r.stdout + r.stderr)
            raise RuntimeError(f"{Path(cmd[0]).name} failed on {src.name}")
        return obj

    with ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        objs = list(ex.map(compile_one, sources()))
    tmp = OUT.with_suffix(f".so.tmp{os.getpid()}")
    subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *map(str, objs), "-o", str(tmp)],
                   check=True)
    os.replace(tmp, OUT)
    return OUT


if __name__ == "__main__":
    print(build(verbose=True))
