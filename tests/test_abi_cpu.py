"""The C ABI on the host, with no GPU: the library loads, exports every
function the headers declare, and reports argument errors before any device
work.  Nothing here enqueues a kernel; the checks that pass validation and
then need a device run only where no device is visible."""

from __future__ import annotations

import ctypes
import glob
import os
import re
import subprocess

import pytest

import transformer_normalization_amd as tn
from transformer_normalization_amd import build as hipbuild

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _lib():
    if not os.path.exists(tn.LIB_PATH):
        hipbuild.build()
    return tn.load_library()


def _no_device_visible() -> bool:
    try:
        import torch
        return torch.cuda.device_count() == 0
    except Exception:
        return True


def declared_functions():
    names = []
    for h in sorted(glob.glob(os.path.join(ROOT, "include", "*.h"))):
        text = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        names += re.findall(r"^\s*[A-Za-z_][\w \*]*?\b(\w+)\s*\([^;{]*\)\s*;", text, flags=re.M)
    return names


def test_headers_declare_the_api():
    names = declared_functions()
    for n in ("rmsnorm_fwd", "rmsnorm_fwd_residual", "rmsnorm_adaln_fwd", "rmsnorm_bwd", "rmsnorm_bwd_workspace_bytes",
              "rmsnorm_status_string", "rmsnorm_last_error", "rmsnorm_tuning_set_geometry",
              "rmsnorm_tuning_set_streaming"):
        assert n in names, n


@pytest.mark.parametrize("name", declared_functions())
def test_library_exports_declared_symbol(name):
    lib = _lib()
    assert hasattr(lib, name), f"{name} is declared but not exported"


def test_status_strings():
    lib = _lib()
    for code, text in tn.STATUS.items():
        assert lib.rmsnorm_status_string(code).decode() == text
    assert lib.rmsnorm_status_string(99).decode() == "RMSN_UNKNOWN_STATUS"


def test_workspace_bytes():
    lib = _lib()
    assert lib.rmsnorm_bwd_workspace_bytes(8192, 6144) == 1024 * 6144 * 4
    assert lib.rmsnorm_bwd_workspace_bytes(100, 4096) == 100 * 4096 * 4
    assert lib.rmsnorm_bwd_workspace_bytes(0, 4096) == 0
    assert lib.rmsnorm_bwd_workspace_bytes(-5, 4096) == 0


def test_argument_errors_need_no_device():
    lib = _lib()
    vp = ctypes.c_void_p
    x, y, w = vp(1 << 32), vp(2 << 32), vp(3 << 32)
    st = lib.rmsnorm_fwd(x, 4096, w, y, 4096, None, 64, 4096, 0.0, tn.RMSN_BF16, tn.RMSN_BF16, None)
    assert st == 1 and b"eps" in lib.rmsnorm_last_error()
    st = lib.rmsnorm_fwd(None, 4096, None, None, 4096, None, 0, 4096, 1e-5, tn.RMSN_BF16, tn.RMSN_BF16, None)
    assert st == 0 and lib.rmsnorm_last_error() == b""
    st = lib.rmsnorm_fwd(x, 4096, w, y, 4096, None, 64, 4096, 1e-5, 5, tn.RMSN_BF16, None)
    assert st == 2


@pytest.mark.skipif(not _no_device_visible(), reason="runs only where no GPU is visible")
def test_c_client():
    """Compile a plain C program against include/ and the library and run it."""
    _lib()
    exe = os.path.join(ROOT, "tests", "c", "abi_check.bin")
    cmd = ["gcc", "-std=c11", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
           "-I", os.path.join(ROOT, "include"), os.path.join(ROOT, "tests", "c", "abi_check.c"), "-o", exe,
           "-L", os.path.dirname(tn.LIB_PATH), "-lrmsnorm", f"-Wl,-rpath,{os.path.dirname(tn.LIB_PATH)}", "-lm"]
    subprocess.run(cmd, check=True)
    try:
        out = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    finally:
        os.remove(exe)
    print(out.stdout)
    assert out.returncode == 0, out.stdout + out.stderr


@pytest.mark.skipif(not _no_device_visible(), reason="runs only where no GPU is visible")
def test_valid_call_without_device_reports_hip_error():
    lib = _lib()
    vp = ctypes.c_void_p
    st = lib.rmsnorm_fwd(vp(1 << 32), 4096, vp(3 << 32), vp(2 << 32), 4096, None, 64, 4096, 1e-5, tn.RMSN_BF16,
                         tn.RMSN_BF16, None)
    assert st == 4, lib.rmsnorm_last_error()
    assert lib.rmsnorm_last_error()


def test_binding_rejects_host_tensors():
    torch = pytest.importorskip("torch")
    x = torch.zeros(4, 8, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="device tensor"):
        tn.rmsnorm_fwd(x)


def test_missing_library_fails_loudly(tmp_path):
    with pytest.raises(ImportError, match="build"):
        tn.load_library(str(tmp_path / "librmsnorm.so"))
