"""The C ABI's host code (argument checks, workspace carving, error messages) built
with AddressSanitizer and driven through every rejection path by a small C program
(tests/asan_abi_driver.c).  Host only: every call fails validation before any HIP
call, so no GPU is touched.  The kernels' objects are linked unchanged."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BUILD = os.path.join(ROOT, "mxfp4_bit_attention_amd", "_build")


def test_c_abi_under_address_sanitizer(tmp_path):
    gxx = shutil.which("g++")
    if gxx is None or not os.path.isdir("/opt/rocm/include"):
        pytest.skip("needs g++ and the ROCm headers")
    objs = [os.path.join(BUILD, f) for f in ("quantize.hip.o", "attention.hip.o")]
    if not all(os.path.exists(o) for o in objs):
        import __graft_entry__
        __graft_entry__.build()
    inc = ["-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROOT, "mxfp4_bit_attention_amd", "csrc"),
           "-I", "/opt/rocm/include", "-D__HIP_PLATFORM_AMD__"]
    # the kernels' objects are linked from copies, so that no compile or link line
    # that carries a sanitizer flag names a HIP source or object
    dev = []
    for o in objs:
        dst = str(tmp_path / os.path.basename(o).replace(".hip.o", "_dev.o"))
        shutil.copyfile(o, dst)
        dev.append(dst)
    api_o = str(tmp_path / "api_asan.o")
    exe = str(tmp_path / "abi_asan")
    subprocess.run([gxx, "-std=c++17", "-O1", "-g", "-Wall", "-fsanitize=address", "-fno-omit-frame-pointer", *inc, "-c",
                    os.path.join(ROOT, "mxfp4_bit_attention_amd", "csrc", "api.cpp"), "-o", api_o], check=True)
    subprocess.run([gxx, "-fsanitize=address", "-g", "-Wall", *inc, "-x", "c", os.path.join(ROOT, "tests", "asan_abi_driver.c"),
                    "-x", "none", api_o, *dev, "-L", "/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib",
                    "-o", exe], check=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120, env=env)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "ok (0 failures)" in r.stdout
