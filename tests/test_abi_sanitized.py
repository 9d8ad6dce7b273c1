"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

api.cpp (argument validation, workspace sizing, error reporting) is rebuilt
for the host with g++ and -fsanitize=address,undefined (device code is not
instrumented: the kernel objects are the ordinary ones), linked into a
second copy of the library, and the CPU ABI tests of test_abi.py are run
against that copy in a child process with the sanitizer runtime preloaded.
Any report aborts the child, so a clean exit means every validation path the
ABI tests take is free of out-of-bounds accesses and undefined behaviour.
"""

import glob
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "block_speculative_decoding_amd")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all"]


def _runtime(name):
    if not shutil.which("g++"):
        return None
    p = subprocess.run(["g++", "-print-file-name=" + name], capture_output=True, text=True).stdout.strip()
    return os.path.realpath(p) if os.path.isabs(p) and os.path.exists(p) else None


def _kernel_objects():
    objs = sorted(o for o in glob.glob(os.path.join(PKG, "_build", "*.o")) if os.path.basename(o) != "api.o")
    if len(objs) < 2:
        from block_speculative_decoding_amd.build import build_library
        build_library(verbose=False)
        objs = sorted(o for o in glob.glob(os.path.join(PKG, "_build", "*.o")) if os.path.basename(o) != "api.o")
    return objs


def test_abi_tests_pass_under_host_sanitizers(tmp_path):
    asan = _runtime("libasan.so")
    if asan is None:
        pytest.skip("g++ with libasan is not available")
    api_o = str(tmp_path / "api_san.o")
    lib = str(tmp_path / "libdflash_san.so")
    cc = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-fPIC"] + SAN + [
        "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", "-I" + os.path.join(ROOT, "include"),
        "-c", os.path.join(PKG, "csrc", "api.cpp"), "-o", api_o]
    r = subprocess.run(cc, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    ld = ["g++", "-shared"] + SAN + ["-o", lib, api_o] + _kernel_objects() + [
        "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib"]
    r = subprocess.run(ld, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr

    env = dict(os.environ)
    env["DFLASH_LIBRARY"] = lib
    env["DFLASH_EXPECT_SANITIZERS"] = "1"
    env["LD_PRELOAD"] = asan
    # The interpreter and torch allocate for the life of the process: leaks
    # are not what this run looks for.
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    r = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_abi.py"), "-x", "-q",
                        "-p", "no:cacheprovider"], cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "ERROR: AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    assert " passed" in r.stdout, out[-2000:]
