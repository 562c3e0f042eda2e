"""Build the plain-C GPU client of the library (tests/c/gpu_client.c) into
tests/c/gpu_client.bin, linked against the in-tree librmsnorm.so (found at
run time next to the package, through an $ORIGIN-relative path) and the HIP
runtime.  Called by the repository's build step; the GPU test runs the
binary it leaves."""

from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
PKG = os.path.join(ROOT, "transformer_normalization_amd")
SRC = os.path.join(HERE, "gpu_client.c")
OUT = os.path.join(HERE, "gpu_client.bin")


def build_gpu_client() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    tmp = f"{OUT}.{os.getpid()}.tmp"
    cmd = ["gcc", "-std=c11", "-O2", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(rocm, "include"), "-I", os.path.join(ROOT, "include"), SRC, "-o", tmp,
           "-L", PKG, "-lrmsnorm", "-L", os.path.join(rocm, "lib"), "-lamdhip64", "-lm",
           "-Wl,-rpath,$ORIGIN/../../transformer_normalization_amd", "-Wl,-rpath," + os.path.join(rocm, "lib")]
    subprocess.run(cmd, check=True)
    os.replace(tmp, OUT)
    return OUT


if __name__ == "__main__":
    print(build_gpu_client())
