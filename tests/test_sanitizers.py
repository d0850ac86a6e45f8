"""CPU sanitizer runs (no GPU): the float64 oracle built with AddressSanitizer
and UndefinedBehaviorSanitizer runs its pins, and the host side of
libpalimpsa (argument validation, workspace planning, status strings; the
kernels are left out of this build) runs the C ABI's invalid-call tables,
each in a subprocess with the sanitizer runtime preloaded.  Any report aborts
the subprocess, which fails the test."""
import glob
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = "/opt/rocm/bin/hipcc"
SAN_ENV = {"ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1:halt_on_error=1",
           "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"}


def _gcc_asan():
    if not shutil.which("gcc"):
        return None
    p = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    return p if os.path.isabs(p) and os.path.exists(p) else None


def _clang_asan():
    found = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return found[-1] if found and os.path.exists(HIPCC) else None


def _run_pytest(args, extra_env, timeout=900):
    env = dict(os.environ, **SAN_ENV, **extra_env)
    env.pop("PYTEST_ADDOPTS", None)
    cmd = [sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", *args]
    res = subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=timeout)
    tail = (res.stdout + res.stderr)[-4000:]
    print(tail)
    assert res.returncode == 0, tail
    assert "ERROR: AddressSanitizer" not in tail and "runtime error:" not in tail, tail
    return tail


@pytest.mark.skipif(_gcc_asan() is None, reason="gcc with libasan not available")
def test_oracle_pins_under_asan_and_ubsan(tmp_path):
    import oracle
    lib = str(tmp_path / "libpalimpsa_oracle_san.so")
    flags = [f for f in oracle.GCC_FLAGS if f != "-O2"]
    subprocess.check_call(["gcc", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
                           "-fno-sanitize-recover=all", *flags, oracle._SRC, "-o", lib, "-lm"])
    tail = _run_pytest(["-m", "not gpu", "tests/test_oracle_pins.py", "tests/test_oracle_bwd_pins.py"],
                       {"PALIMPSA_ORACLE_LIB": lib, "LD_PRELOAD": _gcc_asan()})
    assert " passed" in tail


def _host_san_lib():
    """libpalimpsa with the host code instrumented (the device code is built
    as usual but never launched here), cached by source hash: about a minute
    to build."""
    import hashlib
    import tempfile
    src = os.path.join(ROOT, "bayesian_metaplastic_memory_amd", "csrc", "palimpsa.hip")
    hdr = os.path.join(ROOT, "include", "palimpsa.h")
    key = hashlib.sha256(open(src, "rb").read() + open(hdr, "rb").read()).hexdigest()[:16]
    lib = os.path.join(tempfile.gettempdir(), "libpalimpsa_host_san_%s.so" % key)
    if not os.path.exists(lib):
        tmp = lib + ".tmp%d" % os.getpid()
        subprocess.check_call([HIPCC, "--offload-arch=gfx950", "-O1", "-std=c++17", "-fPIC", "-shared",
                               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-Wno-pass-failed",
                               "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                               "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer",
                               "-I" + os.path.join(ROOT, "include"), src, "-o", tmp],
                              stderr=subprocess.DEVNULL)
        os.replace(tmp, lib)
    return lib


@pytest.mark.skipif(_clang_asan() is None, reason="hipcc or clang's ASan runtime not available")
def test_abi_validation_under_host_asan_and_ubsan():
    lib = _host_san_lib()
    tail = _run_pytest(["-m", "not gpu", "tests/test_abi.py", "-k", "rejects or workspace_size or status"],
                       {"PALIMPSA_TEST_LIB": lib, "LD_PRELOAD": _clang_asan()})
    assert " passed" in tail
