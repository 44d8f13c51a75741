"""The host layer of the library under AddressSanitizer and
UndefinedBehaviorSanitizer, without a GPU.

The library sources are compiled as for the product (gfx950 device code
without sanitizers) with the sanitizers on the host side only, linked with a
C driver
(tests/asan/host_abi_driver.c) that makes the argument-validation calls of
test_abi.py and the HIP-error path of a valid call (no device is visible, so
the launch fails), once as is and once in the checked mode (MLA_DEBUG_SYNC=1);
a sanitizer report or a wrong status fails the test.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "mla_paged_kv_04_amd", "csrc")
SOURCES = ["mla_api.cpp", "mla_kernels.hip", "mla_noalloc.hip"]
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"


@pytest.fixture(scope="module")
def driver(tmp_path_factory):
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not installed")
    out = tmp_path_factory.mktemp("asan")
    objs = []
    common = ["-O1", "-g", "-fno-omit-frame-pointer", "-I", os.path.join(ROOT, "include"),
              "-I", CSRC, "-Xarch_host", "-fsanitize=address",
              "-Xarch_host", "-fsanitize=undefined",
              "-Xarch_host", "-fno-sanitize-recover=undefined"]
    for src in SOURCES:
        obj = str(out / (src + ".o"))
        lang = ["-x", "hip", "--offload-arch=gfx950"] if src.endswith(".hip") else []
        cmd = [HIPCC, "-std=c++17", "-fPIC", *lang, *common, "-c", os.path.join(CSRC, src),
               "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
        assert r.returncode == 0, r.stderr[-3000:]
        objs.append(obj)
    drv_obj = str(out / "driver.o")
    r = subprocess.run(["gcc", "-std=c11", "-O1", "-g", "-fsanitize=address,undefined",
                        "-I", os.path.join(ROOT, "include"), "-c",
                        os.path.join(ROOT, "tests", "asan", "host_abi_driver.c"), "-o", drv_obj],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr[-3000:]
    exe = str(out / "host_abi_driver")
    r = subprocess.run([HIPCC, *objs, drv_obj, "-Xarch_host", "-fsanitize=address",
                        "-Xarch_host", "-fsanitize=undefined", "-o", exe],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-3000:]
    return exe


@pytest.mark.parametrize("debug_sync", ["", "1"])
def test_host_abi_under_sanitizers(driver, debug_sync):
    env = dict(os.environ)
    env["MLA_DEBUG_SYNC"] = debug_sync      # the checked mode's host path too
    # the HIP runtime keeps allocations until exit; leaks are not what this checks
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=0:halt_on_error=1"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    env["HIP_VISIBLE_DEVICES"] = ""
    r = subprocess.run([driver], capture_output=True, text=True, timeout=300, env=env)
    report = r.stdout + r.stderr
    assert "ERROR: AddressSanitizer" not in report, report[-4000:]
    assert "runtime error:" not in report, report[-4000:]
    assert r.returncode == 0, report[-4000:]
    assert "ALL OK" in r.stdout
