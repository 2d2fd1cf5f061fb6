"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU
only): duo_attn.cpp is rebuilt with both sanitizers on its host side, linked with the
ordinary kernel objects and a driver (tests/host_sanitize/abi_driver.cpp) that walks
every argument-validation path returning before a HIP call.  A sanitizer report, or a
return code other than the one the header documents, fails the test."""

import os
import shutil
import subprocess

import pytest

from mixed_head_kv_amd import build as Bld

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OUT = os.path.join(Bld.BUILD, "host_sanitize")
# Sanitizers on the host side only (the device code is built as usual).
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, " ".join(cmd) + "\n" + r.stdout + r.stderr
    return r


@pytest.fixture(scope="module")
def driver():
    hipcc = Bld.hipcc()
    if not os.path.exists(hipcc) and not shutil.which("hipcc"):
        pytest.skip("hipcc not available")
    os.makedirs(OUT, exist_ok=True)
    others = []
    for src in Bld.sources():
        if src == "duo_attn.cpp":
            continue
        obj = os.path.join(Bld.BUILD, os.path.splitext(src)[0] + ".o")
        if not os.path.exists(obj):
            Bld.build()
        others.append(obj)
    flags = [f for f in Bld.HIP_FLAGS if f != "-O3"]
    lib_obj = os.path.join(OUT, "duo_attn_san.o")
    _run([hipcc, *flags, "-O1", "-g", *SAN, "-x", "hip", "-c", os.path.join(Bld.CSRC, "duo_attn.cpp"), "-o", lib_obj])
    drv_obj = os.path.join(OUT, "abi_driver.o")
    _run([hipcc, "-O1", "-g", "-std=c++17", *SAN, "-x", "c++", "-c",
          os.path.join(ROOT, "tests", "host_sanitize", "abi_driver.cpp"), "-o", drv_obj])
    exe = os.path.join(OUT, "abi_driver_san")
    _run([hipcc, f"--offload-arch={Bld.ARCH}", *SAN, drv_obj, lib_obj, *others, "-o", exe])
    return exe


def test_validation_paths_are_clean_under_asan_and_ubsan(driver):
    env = dict(os.environ)
    env["ASAN_OPTIONS"] = "halt_on_error=1:detect_leaks=1:abort_on_error=0"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    env["HIP_VISIBLE_DEVICES"] = ""  # (no device is ever needed by these paths)
    r = subprocess.run([driver], capture_output=True, text=True, env=env, timeout=120)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out
    assert "runtime error" not in out and "AddressSanitizer" not in out, out
    assert "ok: 0 failure(s)" in r.stdout, out
