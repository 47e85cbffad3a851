"""Build libfa.so (HIP kernels for gfx950 + the C ABI) in this package
directory with hipcc."""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libfa.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

SOURCES = ["table.cpp", "api.cpp", "emission.hip", "tree.hip", "sample.hip", "marginals.hip",
           "commit.hip", "noalloc.hip", "probe.hip", "map.hip",
           "chain.hip", "live.hip"]

COMMON = ["-O3", "-fPIC", "-std=c++17", "-Wall", f"-I{CSRC}"]
# packed fp32 instructions are kept out of every gfx950 code object
DEVICE = [f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-fno-gpu-rdc"]


def _obj(src: str, build_dir: str) -> str:
    return os.path.join(build_dir, src.rsplit(".", 1)[0] + ".o")


def _compile(src: str, build_dir: str) -> str:
    out = _obj(src, build_dir)
    path = os.path.join(CSRC, src)
    cmd = [HIPCC] + COMMON
    cmd += (["-x", "hip"] + DEVICE) if src.endswith(".hip") else ["-D__HIP_PLATFORM_AMD__"]
    cmd += ["-c", path, "-o", out]
    subprocess.run(cmd, check=True)
    return out


def build(verbose: bool = False) -> str:
    build_dir = os.path.join(HERE, "_build")
    os.makedirs(build_dir, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(6, os.cpu_count() or 1)) as ex:
        objs = list(ex.map(lambda s: _compile(s, build_dir), SOURCES))
    tmp = LIB + ".tmp"
    subprocess.run([HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + objs
                   + ["-lamdhip64"], check=True)
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
