"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer, on the CPU.

* The oracle (plain C) is built with gcc's ASan and UBSan (float-cast and
  divide-by-zero checks included) together with tests/c/oracle_sanitize.c,
  which drives every oracle routine over random ragged shapes held in
  exactly sized heap buffers, and every 16-bit pattern through the codecs.
* The library's host code (argument checks, overlap and size arithmetic,
  geometry choice, the device query) is built with hipcc, the sanitizers on
  the host side only (each -fsanitize flag behind -Xarch_host; the device
  code is compiled exactly as in the product), and driven from C by
  tests/c/abi_check.c (every documented rejection) and tests/c/abi_fuzz.c
  (random extreme arguments to every entry point).

The library runs are skipped where a device is visible: there a call that
passes every check would launch a kernel on the fake addresses.  Any
sanitizer report aborts the program (-fno-sanitize-recover=all), which fails
the test with the report in its output.
"""

from __future__ import annotations

import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

from tests.test_abi_cpu import _no_device_visible

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
CLANG = os.path.join(ROCM, "llvm", "bin", "clang")
HOST_SANITIZE = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                 "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")


def _run(cmd, **kw):
    out = subprocess.run(cmd, capture_output=True, text=True, env=ENV, **kw)
    return out.returncode, out.stdout + out.stderr


def test_oracle_under_sanitizers(tmp_path):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not found")
    exe = str(tmp_path / "oracle_sanitize")
    cmd = ["gcc", "-std=c11", "-O1", "-g", "-Wall", "-Wextra", "-Werror", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined,float-cast-overflow,float-divide-by-zero", "-fno-sanitize-recover=all",
           os.path.join(ROOT, "tests", "c", "oracle_sanitize.c"), os.path.join(ROOT, "oracle", "rmsnorm_oracle.c"),
           "-o", exe, "-lm"]
    subprocess.run(cmd, check=True)
    rc, out = _run([exe, "400"], timeout=300)
    print(out)
    assert rc == 0, out


@pytest.fixture(scope="module")
def sanitized_library(tmp_path_factory):
    if not _no_device_visible():
        pytest.skip("runs only where no GPU is visible")
    if not (os.path.exists(CLANG) and os.path.exists(os.path.join(ROCM, "bin", "hipcc"))):
        pytest.skip("ROCm clang/hipcc not found")
    from transformer_normalization_amd import build

    d = tmp_path_factory.mktemp("sanitized")
    flags = build.compile_flags()

    def compile_one(src):
        obj = str(d / (os.path.splitext(src)[0] + ".o"))
        subprocess.run([build.hipcc(), *flags, *HOST_SANITIZE, "-c", os.path.join(build.CSRC, src), "-o", obj],
                       check=True, capture_output=True)
        return obj

    with ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as pool:
        objs = list(pool.map(compile_one, build.SOURCES))
    lib = str(d / "librmsnorm.so")
    subprocess.run([build.hipcc(), f"--offload-arch={build.ARCH}", "-shared", "-fPIC", *HOST_SANITIZE[:4],
                    "-shared-libsan", *objs, "-o", lib], check=True, capture_output=True)
    return d


def _client(lib_dir, source, name):
    runtime = subprocess.run([CLANG, "--print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True,
                             text=True, check=True).stdout.strip()
    exe = str(lib_dir / name)
    cmd = [CLANG, "-std=c11", "-O1", "-g", "-Wall", "-Wextra", "-Werror", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", "-shared-libsan", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROCM, "include"),
           "-I", os.path.join(ROOT, "include"), os.path.join(ROOT, "tests", "c", source), "-o", exe,
           "-L", str(lib_dir), "-lrmsnorm", "-L", os.path.join(ROCM, "lib"), "-lamdhip64",
           f"-Wl,-rpath,{lib_dir}", f"-Wl,-rpath,{os.path.dirname(runtime)}", f"-Wl,-rpath,{os.path.join(ROCM, 'lib')}",
           "-lm"]
    subprocess.run(cmd, check=True)
    return exe


def test_abi_rejections_under_sanitizers(sanitized_library):
    exe = _client(sanitized_library, "abi_check.c", "abi_check")
    rc, out = _run([exe], timeout=300)
    print(out)
    assert rc == 0, out


@pytest.mark.parametrize("seed", [1, 2, 3])
def test_abi_fuzz_under_sanitizers(sanitized_library, seed):
    exe = str(sanitized_library / "abi_fuzz")
    if not os.path.exists(exe):
        exe = _client(sanitized_library, "abi_fuzz.c", "abi_fuzz")
    rc, out = _run([exe, "100000", str(seed)], timeout=300)
    print(out)
    assert rc == 0, out
