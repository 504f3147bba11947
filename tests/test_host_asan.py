"""Phase 1 under AddressSanitizer (CPU only).

The host planner (``fa_plan.cpp``) is compiled with g++ and
``-fsanitize=address`` into a stand-alone library, with host stubs for the
device entry points (``tests/asan_stub.cpp``), and the phase-1 tests of
``test_abi_host.py`` run against it in a child process with the sanitizer
runtime preloaded.  Any out-of-bounds access or use-after-free in
validation, planning, describe, destroy or merge validation fails the run.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "attention_forward_fa_amd", "csrc")
OUT = os.path.join(ROOT, "_build", "asan")

# tests that need the device half (phase 2, the clock probe) or the full export list are left out
DESELECT = "not phase2 and not not_consumed and not clock_probe and not header_symbols and not noalloc"


def _asan_runtime():
    r = subprocess.run(["g++", "-print-file-name=libasan.so"], stdout=subprocess.PIPE, text=True)
    path = r.stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


@pytest.fixture(scope="module")
def asan_lib():
    rt = _asan_runtime()
    if rt is None:
        pytest.skip("g++ has no AddressSanitizer runtime here")
    os.makedirs(OUT, exist_ok=True)
    lib = os.path.join(OUT, "libfa_fwd_asan.so")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address", "-fPIC", "-shared",
           "-I", os.path.join(ROOT, "include"), "-I", CSRC, os.path.join(CSRC, "fa_plan.cpp"),
           os.path.join(ROOT, "tests", "asan_stub.cpp"), "-o", lib]
    subprocess.run(cmd, check=True)
    return lib, rt


def test_phase1_under_asan(asan_lib):
    lib, rt = asan_lib
    env = dict(os.environ, FA_FWD_LIB=lib, LD_PRELOAD=rt, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0")
    env.pop("FA_FWD_KERNEL", None)
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi_host.py"), "-k", DESELECT],
                       cwd=ROOT, env=env, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, timeout=600)
    assert "AddressSanitizer" not in r.stdout, r.stdout[-4000:]
    assert r.returncode == 0, r.stdout[-4000:]
    assert " passed" in r.stdout, r.stdout[-2000:]
