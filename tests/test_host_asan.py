"""The C-ABI's host-side argument handling under AddressSanitizer (CPU; no
GPU is touched).  The library's sources are compiled with the sanitizer on
their host code only (-Xarch_host before -fsanitize; device code is built as
usual, so the objects link) into a temporary directory, linked with
tests/host_checks.cpp, and run: every entry point's argument checks
(invalid arguments, unsupported shapes and descriptor spans, empty problems,
the allocation-free dispatch's scratch limit) must return the documented
status before any device work, with no sanitizer report."""

import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

from fp8_routed_expert_amd import build as lib_build

HERE = os.path.dirname(os.path.abspath(__file__))
CLANG = "/opt/rocm/lib/llvm/bin/clang++"
ROCM_LIB = "/opt/rocm/lib"


def test_host_argument_checks_under_asan(tmp_path):
    if not (os.path.exists(lib_build.HIPCC) and os.path.exists(CLANG)):
        pytest.skip("ROCm compilers not installed")
    srcs = sorted(os.path.join(lib_build.CSRC, f) for f in os.listdir(lib_build.CSRC)
                  if f.endswith(".hip"))
    flags = [f for f in lib_build.FLAGS if f != "-O3"] + ["-O1", "-g", "-Xarch_host",
                                                          "-fsanitize=address"]

    def compile_one(src):
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        r = subprocess.run([lib_build.HIPCC, *flags, "-c", src, "-o", obj],
                           capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-2000:]
        return obj

    with ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(compile_one, srcs))
    main_o = str(tmp_path / "host_checks.o")
    r = subprocess.run([CLANG, "-O1", "-g", "-std=c++17", "-fsanitize=address",
                        f"-I{lib_build.INCLUDE}", "-c", os.path.join(HERE, "host_checks.cpp"),
                        "-o", main_o], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    exe = str(tmp_path / "host_checks")
    r = subprocess.run([CLANG, "-fsanitize=address", main_o, *objs, f"-L{ROCM_LIB}",
                        "-lamdhip64", f"-Wl,-rpath,{ROCM_LIB}", "-o", exe],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=0")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert "host checks: 0 failures" in out, out[-2000:]
