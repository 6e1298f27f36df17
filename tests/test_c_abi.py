"""The C ABI from plain C: tests/c_abi_consumer.c is compiled with gcc against
include/a2av.h and linked to liba2av.so (a CPU test: the header is C-clean and
the library links), then run on the GPU (a GPU test)."""
import os
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIBDIR = os.path.join(ROOT, "embeddings_a2av_virtual_amd")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def _build(tmp_path):
    exe = tmp_path / "c_abi_consumer"
    cmd = ["gcc", "-std=c11", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
           f"-I{os.path.join(ROOT, 'include')}", f"-I{ROCM}/include",
           os.path.join(HERE, "c_abi_consumer.c"), "-o", str(exe),
           f"-L{LIBDIR}", "-la2av", f"-L{ROCM}/lib", "-lamdhip64",
           f"-Wl,-rpath,{LIBDIR}", f"-Wl,-rpath,{ROCM}/lib"]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    return exe


def test_c_consumer_compiles_and_links(tmp_path):
    assert os.path.exists(os.path.join(LIBDIR, "liba2av.so")), "build the library first"
    exe = _build(tmp_path)
    assert exe.exists()


@pytest.mark.gpu
def test_c_consumer_runs(tmp_path):
    exe = _build(tmp_path)
    p = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert p.returncode == 0, p.stdout + p.stderr
    assert "c abi consumer: ok" in p.stdout
