"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

abi.hip (argument checks, the CSR transpose and the budget allocation, which
read caller arrays on the host) is rebuilt with the sanitizers on its host
side only, linked with the other objects of the library build and a driver
(tests/host_sanitize_driver.cpp) that calls those entry points with exact-size
heap buffers.  CPU only: nothing here launches a kernel.
"""
import glob
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "wht_adapters_amd")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
SAN_HOST = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]


@pytest.fixture(scope="module")
def driver(tmp_path_factory):
    objs = sorted(o for o in glob.glob(os.path.join(PKG, "_build", "*.o")) if not o.endswith("abi.hip.o"))
    if not os.path.exists(HIPCC) or shutil.which("g++") is None or not objs:
        pytest.skip("needs hipcc, g++ and the library's object files (run the build first)")
    d = tmp_path_factory.mktemp("san")
    inc = "-I" + os.path.join(ROOT, "include")
    abi_o, drv_o, exe = str(d / "abi_san.o"), str(d / "driver.o"), str(d / "driver")
    steps = [
        [HIPCC, "-std=c++17", "-O1", "-g", "-fPIC", "--offload-arch=gfx950", "-Xclang", "-target-feature",
         "-Xclang", "-packed-fp32-ops", *SAN_HOST, inc, "-c", os.path.join(PKG, "csrc", "abi.hip"), "-o", abi_o],
        ["g++", "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
         "-fno-omit-frame-pointer", inc, "-c", os.path.join(ROOT, "tests", "host_sanitize_driver.cpp"), "-o", drv_o],
        [HIPCC, "--offload-arch=gfx950", "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
         drv_o, abi_o, *objs, "-o", exe],
    ]
    for cmd in steps:
        p = subprocess.run(cmd, capture_output=True, text=True)
        assert p.returncode == 0, p.stderr[-4000:]
    return exe


def _run(exe, *args):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1",
               HIP_VISIBLE_DEVICES="")
    return subprocess.run([exe, *args], capture_output=True, text=True, timeout=120, env=env)


def test_host_entry_points_clean_under_sanitizers(driver):
    p = _run(driver)
    assert p.returncode == 0, p.stdout[-3000:] + p.stderr[-3000:]
    assert "0 failure(s)" in p.stdout
    assert "Sanitizer" not in p.stderr and "runtime error" not in p.stderr


def test_sanitizer_is_live(driver):
    """An output array one element short must be reported (instrumented build)."""
    p = _run(driver, "--short-output")
    assert p.returncode != 0
    assert "heap-buffer-overflow" in p.stderr
