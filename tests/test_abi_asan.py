"""The C ABI's host code under AddressSanitizer (CPU only, no device needed).

The library's sources are compiled for gfx950 as in the release build, with the host half
instrumented by ASan; a native driver (tests/native/abi_asan_driver.cpp) calls every entry point
with invalid arguments (validation paths, messages, workspace arithmetic), runs the host
precondition check on 2,000 random tables against a reference written out in the driver, and
checks that the error message is per thread.  Any host memory error fails the test.
"""
import concurrent.futures
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "paged_mla_latent_amd", "csrc")
SOURCES = ["mla_api.hip", "decode.hip", "decode_wide.hip", "merge.hip", "cache_write.hip", "gather.hip"]
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"


def _run(cmd):
    p = subprocess.run(cmd, capture_output=True, text=True)
    assert p.returncode == 0, f"{' '.join(cmd)}\n{p.stdout}\n{p.stderr}"


@pytest.fixture(scope="module")
def driver(tmp_path_factory):
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc is not available")
    out = tmp_path_factory.mktemp("asan")
    common = ["--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC",
              "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
              "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer",
              "-I", os.path.join(ROOT, "include"), "-I", CSRC]
    objs = [str(out / (os.path.splitext(s)[0] + ".o")) for s in SOURCES]
    cmds = [[HIPCC, *common, "-c", os.path.join(CSRC, s), "-o", o] for s, o in zip(SOURCES, objs)]
    with concurrent.futures.ThreadPoolExecutor(max_workers=6) as ex:
        list(ex.map(_run, cmds))
    drv = str(out / "abi_asan_driver.o")
    _run([HIPCC, *common, "-c", os.path.join(ROOT, "tests", "native", "abi_asan_driver.cpp"), "-o", drv])
    exe = str(out / "abi_asan_driver")
    _run([HIPCC, "--offload-arch=gfx950", "-Xarch_host", "-fsanitize=address", drv, *objs, "-o", exe])
    return exe


def test_abi_host_code_is_clean_under_asan(driver):
    # the host half of the C ABI really is instrumented (its loads and stores report to ASan)
    syms = subprocess.run(["nm", os.path.join(os.path.dirname(driver), "mla_api.o")], capture_output=True,
                          text=True).stdout
    assert "__asan_report_load" in syms or "__asan_report_store" in syms
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0:halt_on_error=1")
    p = subprocess.run([driver], capture_output=True, text=True, env=env, timeout=300)
    assert "AddressSanitizer" not in p.stderr, p.stderr[-4000:]
    assert p.returncode == 0, p.stdout + p.stderr[-4000:]
    assert "all checks passed" in p.stdout
