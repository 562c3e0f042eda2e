"""Build librmsnorm.so (the gfx950 HIP library) in-tree with hipcc.

    python -m transformer_normalization_amd.build

Every kernel is compiled for gfx950 only, with float32/float16 denormals kept
and packed-float32 instruction selection switched off.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys
import time

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "librmsnorm.so")
SOURCES = ["host_common.hip", "rmsnorm_api.hip", "kernels_fwd.hip", "kernels_fwd_residual.hip", "kernels_adaln.hip", "kernels_bwd.hip",
           "kernels_bwd_residual.hip", "kernels_bwd_mis.hip", "kernels_fwd_mis.hip", "rope_api.hip", "kernels_rope.hip", "kernels_ln.hip", "kernels_ln_mis.hip",
           "kernels_copy.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (set HIPCC or install ROCm under /opt/rocm)")


def compile_flags() -> list[str]:
    return [
        f"--offload-arch={ARCH}",
        "-O3",
        "-std=c++17",
        "-fPIC",
        "-fvisibility=hidden",
        "-Wall",
        "-Werror",
        "-Wno-unused-command-line-argument",
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-I", INCLUDE,
        "-I", CSRC,
    ]


def build(verbose: bool = False) -> str:
    """Compile the library (always; callers decide whether a rebuild is needed)."""
    objs = []
    t0 = time.time()
    procs = []
    for src in SOURCES:
        obj = os.path.join(CSRC, os.path.splitext(src)[0] + ".o")
        cmd = [hipcc(), *compile_flags(), "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((subprocess.Popen(cmd), cmd))
        objs.append(obj)
    for p, cmd in procs:
        if p.wait() != 0:
            raise RuntimeError(f"compile failed: {' '.join(cmd)}")
    tmp = LIB + ".tmp"
    link = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(link), flush=True)
    subprocess.run(link, check=True)
    os.replace(tmp, LIB)
    for o in objs:
        os.remove(o)
    if verbose:
        print(f"built {LIB} in {time.time() - t0:.1f}s", flush=True)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
