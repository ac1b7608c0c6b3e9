"""The C ABI's host code under the address and undefined-behaviour sanitizers (CPU only).

Builds the library once more with ``-Xarch_host -fsanitize=address,undefined``
(host code instrumented; the gfx950 device code is compiled as usual) into a
temporary directory, links ``abi_host_checks.cpp`` against it, and runs that
program on the CPU: workspace-size queries over every path's planner and
every documented rejection of invalid arguments. Nothing is launched. Any
sanitizer report fails the test.
"""
from __future__ import annotations

import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "block_sparse_long_compress_amd", "csrc")
INCLUDE = os.path.join(ROOT, "include")


def _hipcc():
    path = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc")
    return path if os.path.exists(path) else shutil.which("hipcc")


SANITIZE = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]


@pytest.mark.skipif(_hipcc() is None, reason="hipcc not available")
def test_abi_host_code_under_sanitizers(tmp_path):
    import importlib.util

    spec = importlib.util.spec_from_file_location("qsa_build", os.path.join(ROOT, "block_sparse_long_compress_amd",
                                                                            "build.py"))
    build = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(build)
    hipcc = _hipcc()
    flags = [f for f in build.compile_flags() if f != "-Wall"] + ["-g", "-O1"] + SANITIZE

    def compile_one(src):
        obj = str(tmp_path / (os.path.splitext(src)[0] + ".o"))
        cmd = [hipcc, *flags, *build.EXTRA_FLAGS.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, f"{src}: {r.stderr[-2000:]}"
        return obj

    with ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        objs = list(ex.map(compile_one, build.SOURCES))
    lib = str(tmp_path / "libqsa_san.so")
    r = subprocess.run([hipcc, "-shared", "-fPIC", f"--offload-arch={build.ARCH}", *SANITIZE, "-o", lib, *objs],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    exe = str(tmp_path / "abi_host_checks")
    # the driver links with the same compiler, so that its sanitizer runtime serves the library too
    clang = os.path.join(os.path.dirname(os.path.realpath(hipcc)), "..", "llvm", "bin", "clang++")
    clang = clang if os.path.exists(clang) else os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "llvm", "bin",
                                                             "clang++")
    r = subprocess.run([clang, "-std=c++17", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
                        "-I", INCLUDE, os.path.join(ROOT, "tests", "abi_host_checks.cpp"), lib,
                        f"-Wl,-rpath,{tmp_path}", "-o", exe], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=600)
    report = r.stdout + r.stderr
    assert r.returncode == 0, report[-4000:]
    assert "ERROR: AddressSanitizer" not in report and "runtime error" not in report, report[-4000:]
    assert report.strip().startswith("ok:"), report[-2000:]
