"""The library's host code (descriptor validation, planning, workspace sizing,
the schedule) under AddressSanitizer and UndefinedBehaviorSanitizer, on the
CPU: the library is rebuilt with both sanitizers on its host side only (the
device code is the ordinary gfx950 build) and the ABI checks run against it
in a child process with the sanitizer runtime preloaded.  Any report, or any
undefined behaviour (recovery off), fails the run."""
import glob
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

import pytest

from second_order_optimizer_amd import build as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN_DIR = os.path.join(B.OBJ, "hostsan")
SAN_LIB = os.path.join(SAN_DIR, "libkfac_hostsan.so")
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined"]


def _build() -> str:
    os.makedirs(SAN_DIR, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(B.CSRC, "*.hip")))
    flags = [f for f in B.HIP_FLAGS if f != "-O3"] + ["-O1", "-g", "-fno-omit-frame-pointer"] + SAN + [
        "-Xarch_host", "-fno-sanitize-recover=undefined"]
    objs = [os.path.join(SAN_DIR, os.path.basename(s)[:-4] + ".o") for s in srcs]
    with ThreadPoolExecutor(max(1, min(8, len(srcs)))) as ex:
        list(ex.map(lambda so: B._run([B.HIPCC] + flags + ["-c", so[0], "-o", so[1]], False), zip(srcs, objs)))
    B._run([B.HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC"] + SAN + ["-o", SAN_LIB] + objs, False)
    return SAN_LIB


def _asan_runtime() -> str:
    r = subprocess.run([B.HIPCC, "-print-file-name=libclang_rt.asan-x86_64.so"], stdout=subprocess.PIPE,
                       stderr=subprocess.DEVNULL, text=True)
    return r.stdout.strip()


@pytest.mark.skipif(not os.path.exists(B.HIPCC), reason="hipcc not installed")
def test_abi_checks_under_asan_and_ubsan():
    rt = _asan_runtime()
    if not os.path.isabs(rt) or not os.path.exists(rt):
        pytest.skip("clang AddressSanitizer runtime not found")
    lib = _build()
    env = dict(os.environ, KFAC_LIBRARY=lib, LD_PRELOAD=rt, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", "-m", "not gpu",
                        os.path.join(ROOT, "tests", "test_abi.py")],
                       cwd=ROOT, env=env, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, timeout=600)
    out = r.stdout
    assert r.returncode == 0, out[-4000:]
    assert "AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    assert " passed" in out and " failed" not in out, out[-2000:]
