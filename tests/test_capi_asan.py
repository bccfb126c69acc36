"""The C ABI's host code under AddressSanitizer (CPU only, no GPU needed).

capi.cpp (argument validation, workspace sizing, the wire-format layout and every
host-side branch of the entry points) is rebuilt with g++ -fsanitize=address and
linked with the library's other objects into a separate libgc.so; test_capi.py then
runs against that build in a child process with the sanitizer runtime preloaded.
Any heap or stack error in the host code aborts the child and fails this test.
"""
import os
import shutil
import subprocess
import sys

import pytest

from gc_testlib import ROOT, ensure_built

CSRC = os.path.join(ROOT, "gradient_compression_ddp_amd", "csrc")
BUILD = os.path.join(ROOT, "gradient_compression_ddp_amd", "_build")
OBJS = ["minmax.o", "qsgd.o", "terngrad.o", "ef_topk.o", "powersgd.o", "decompress.o", "noalloc.o"]


def test_capi_under_asan(tmp_path):
    gxx = shutil.which("g++")
    if not gxx or not os.path.exists("/opt/rocm/include/hip/hip_runtime.h"):
        pytest.skip("g++ or the HIP headers are not available")
    asan = subprocess.run([gxx, "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    if not os.path.isabs(asan) or not os.path.exists(asan):
        pytest.skip("the g++ AddressSanitizer runtime is not installed")
    ensure_built()
    objs = [os.path.join(BUILD, o) for o in OBJS]
    if not all(os.path.exists(o) for o in objs):
        pytest.skip("the library's objects are not built")
    obj = str(tmp_path / "capi_asan.o")
    lib = str(tmp_path / "libgc.so")
    subprocess.run([gxx, "-std=c++17", "-O1", "-g", "-fPIC", "-fsanitize=address", "-fno-omit-frame-pointer",
                    "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", f"-I{os.path.join(ROOT, 'include')}",
                    f"-I{CSRC}", "-c", os.path.join(CSRC, "capi.cpp"), "-o", obj], check=True)
    subprocess.run([gxx, "-shared", "-fsanitize=address", "-o", lib, obj] + objs +
                   ["-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib"], check=True)
    env = dict(os.environ, GC_LIB_PATH=lib, LD_PRELOAD=asan,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1:halt_on_error=1")
    res = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                          os.path.join(ROOT, "tests", "test_capi.py")],
                         cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert res.returncode == 0, res.stdout[-3000:] + res.stderr[-3000:]
    assert "AddressSanitizer" not in res.stderr, res.stderr[-3000:]
