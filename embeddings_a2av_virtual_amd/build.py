"""Build ``liba2av.so`` in-tree with hipcc for gfx950.

``python -m embeddings_a2av_virtual_amd.build`` compiles every HIP source under
``csrc/`` into one shared library next to this file. hipcc cross-compiles
without a GPU.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "liba2av.so")
SOURCES = ["a2av.hip", "moe.hip", "blocks.hip"]
ARCH = "gfx950"

FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-fvisibility=hidden",
    "-Wall",
    # fp32 subnormals kept: the combine's results are defined bit for bit
    "-fno-gpu-flush-denormals-to-zero",
    # packed fp32 instructions are kept out of every kernel
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # the first five kernel arguments arrive in scalar registers at wave
    # launch (kernels whose leading arguments are pointers and sizes skip a
    # memory round trip before their first load)
    "-mllvm", "-amdgpu-kernarg-preload-count=5",
    f"-I{os.path.join(ROOT, 'include')}",
]


def build(out: str = LIB, extra: tuple = (), verbose: bool = False) -> str:
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    tmp = out + ".tmp"
    cmd = [hipcc, *FLAGS, *extra, "-o", tmp, *srcs]
    if verbose:
        print(" ".join(cmd), flush=True)
    p = subprocess.run(cmd, capture_output=True, text=True)
    if p.returncode != 0:
        sys.stderr.write(p.stdout + p.stderr)
        raise RuntimeError(f"hipcc failed ({p.returncode})")
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
