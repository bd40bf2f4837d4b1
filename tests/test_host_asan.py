"""The library's host code under AddressSanitizer (CPU only).

Builds a second copy of libmla with AddressSanitizer on the host side only
(the device code is compiled as usual) and runs tests/host_asan/driver.cpp
against it: sizing and layout queries, workspace fits and every argument
check that returns before a launch.  Any invalid host memory access in that
code (validation, planners, workspace layout) stops the driver with an
AddressSanitizer report.  Leak checking is off: the HIP runtime keeps
allocations of its own for the life of the process.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "head_latent_attention_13_amd", "csrc")
ROCM = "/opt/rocm"


def _tools():
    hipcc = os.path.join(ROCM, "bin", "hipcc")
    clang = os.path.join(ROCM, "llvm", "bin", "clang++")
    if not (os.path.exists(hipcc) and os.path.exists(clang)):
        pytest.skip("ROCm compilers not found")
    return hipcc, clang


def test_host_code_under_address_sanitizer(tmp_path):
    hipcc, clang = _tools()
    from head_latent_attention_13_amd.build import SOURCES
    lib = str(tmp_path / "libmla_asan.so")
    host_asan = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer"]
    cmd = [hipcc, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", "-shared",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-Wno-pass-failed", *host_asan,
           "-o", lib, *[os.path.join(CSRC, s) for s in SOURCES]]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=900)
    assert r.returncode == 0, r.stderr[-3000:]
    # the host code is instrumented (its objects call into the sanitizer runtime)
    nm = subprocess.run([shutil.which("nm") or "nm", "-D", "--undefined-only", lib],
                        capture_output=True, text=True, timeout=60)
    assert "__asan_report_load" in nm.stdout
    exe = str(tmp_path / "driver")
    r = subprocess.run([clang, "-fsanitize=address", "-fno-omit-frame-pointer", "-g", "-O1", "-std=c++17",
                        "-I", os.path.join(ROOT, "include"), os.path.join(ROOT, "tests", "host_asan", "driver.cpp"),
                        lib, "-Wl,-rpath," + str(tmp_path), "-o", exe], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-3000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0", HIP_VISIBLE_DEVICES="")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert "host checks: 0 failures" in out
