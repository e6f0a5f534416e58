"""The host side of libkvr under AddressSanitizer and UndefinedBehaviorSanitizer
(CPU only).  Every library source is compiled with both sanitizers on its host
side (the device code is built but never runs) and linked with tests/abi_sanitize.cpp, which
calls each C entry point with arguments that must be rejected before any
device work, plus a few that reach the HIP runtime and must come back as
KVR_ERR_HIP on a machine without a GPU.  A sanitizer report or a wrong
status fails the test."""
import glob
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "packed_partial_prefill_amd", "csrc")
OUT = os.path.join(ROOT, "_build", "abi_sanitize")


def _hipcc():
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    pytest.skip("hipcc not available")


def _compile(src, obj):
    # the device code is built as for the library (never run here); each
    # -fsanitize= applies to the host compilation only
    cmd = [_hipcc(), "-x", "hip", "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC",
           "-fno-omit-frame-pointer", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    return obj


@pytest.mark.slow
def test_host_validation_under_asan_and_ubsan():
    os.makedirs(OUT, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    jobs = [(s, os.path.join(OUT, os.path.basename(s) + ".o")) for s in srcs]
    jobs.append((os.path.join(ROOT, "tests", "abi_sanitize.cpp"), os.path.join(OUT, "driver.o")))
    from concurrent.futures import ThreadPoolExecutor
    with ThreadPoolExecutor(min(8, len(jobs))) as ex:
        objs = list(ex.map(lambda j: _compile(*j), jobs))
    exe = os.path.join(OUT, "abi_sanitize")
    cmd = [_hipcc(), "--offload-arch=gfx950", "-Xarch_host", "-fsanitize=address",
           "-Xarch_host", "-fsanitize=undefined", "-o", exe, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    env = dict(os.environ)
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1:abort_on_error=0"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    env["HIP_VISIBLE_DEVICES"] = ""     # never touch a GPU, even where there is one
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    out = r.stdout + r.stderr
    assert "ERROR: AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert " 0 failed" in r.stdout, out[-4000:]
