"""The library's host code (argument validation, workspace planning, the
ABI's error paths) under AddressSanitizer and UndefinedBehaviorSanitizer.

Every csrc/*.hip file is compiled with the sanitizers on the host side only
(the device code is built unoptimised, to keep the build short, and is never
launched), and linked with tests/host_asan/host_check.cpp, which drives every
entry point over a grid of shapes and bad arguments without touching a GPU
(see that file).  CPU only; about a minute of compilation."""

import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "sparse_long_context_ekv_amd", "csrc")
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-fno-sanitize-recover=undefined"]


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return r


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not installed")
def test_host_code_under_address_and_ub_sanitizers(tmp_path):
    srcs = sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))
    common = ["-std=c++17", "-O1", "-g", "-fPIC", "--offload-arch=gfx950", "-Xarch_device", "-O0", "-Xarch_device", "-g0",
              f"-I{os.path.join(ROOT, 'include')}"] + SAN

    def compile_one(src):
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        _run([HIPCC, *common, "-c", src, "-o", obj])
        return obj

    with ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(compile_one, srcs))
    drv = str(tmp_path / "host_check.o")
    _run([HIPCC, *common, "-c", os.path.join(ROOT, "tests", "host_asan", "host_check.cpp"), "-o", drv])
    exe = str(tmp_path / "host_check")
    _run([HIPCC, *SAN, drv, *objs, "-o", exe])
    syms = subprocess.run(["nm", exe], capture_output=True, text=True).stdout
    assert "__asan_report_load" in syms and "__ubsan_handle" in syms     # the checks are really compiled in
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=600)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "host checks passed" in r.stdout
    assert "ERROR: AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr, r.stderr
