"""The C ABI used from plain C on the GPU: tests/c/gpu_client.c allocates
with hipMalloc, calls rmsnorm_fwd, rmsnorm_fwd_residual and rope_apply on
its own stream and checks exact closed-form results (no Python or torch in
that process).  The binary is built by the repository's build step."""

from __future__ import annotations

import os
import subprocess

import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

EXE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c", "gpu_client.bin")


def test_plain_c_client_on_the_gpu():
    assert os.path.exists(EXE), f"{EXE} is missing: run __graft_entry__.build() (or python tests/c/build.py)"
    p = subprocess.run([EXE], capture_output=True, text=True, timeout=120)
    print(p.stdout)
    assert p.returncode == 0, p.stdout + p.stderr
    assert p.stdout.strip().endswith("ok (0 failures)")
