"""The oracle and the library's host code under AddressSanitizer and
UndefinedBehaviorSanitizer, on the CPU.

The oracle is rebuilt with gcc's address and undefined-behaviour checks and
its pins and parity-rule tests run against it in a child process; the HIP
library is rebuilt with the checks on its host code only (argument
validation, the path predicate, record building) and the ABI tests that need
no GPU run against it.  Any report aborts the child, which fails the test.
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = "/opt/rocm/bin/hipcc"


def _child(env_extra, args, timeout):
    env = dict(os.environ)
    env.update(env_extra)
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1:halt_on_error=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    cmd = [sys.executable, "-m", "pytest", "-q", "-x", "-s", "-p", "no:cacheprovider", "-m", "not gpu", *args]
    res = subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=timeout)
    out = res.stdout + res.stderr
    assert res.returncode == 0, out[-4000:]
    assert "ERROR: AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    return out


def test_oracle_under_asan_and_ubsan(tmp_path):
    import oracle
    if shutil.which("gcc") is None:
        pytest.skip("gcc missing")
    asan = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    if not os.path.isabs(asan):
        pytest.skip("gcc has no libasan")
    lib = str(tmp_path / "oracle_san.so")
    flags = [f for f in oracle.GCC_FLAGS if f != "-O2"]
    subprocess.check_call(["gcc", *flags, "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address",
                           "-fsanitize=undefined", "-fno-sanitize-recover=all",
                           os.path.join(ROOT, "oracle", "sampler_oracle.c"), "-o", lib, "-lm"])
    _child({"LD_PRELOAD": asan, "ORACLE_LIBRARY": lib},
           ["tests/test_oracle_pins.py", "tests/test_parity_rules.py"], timeout=900)


def test_library_host_code_under_asan_and_ubsan(tmp_path):
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc missing")
    rt = subprocess.run([HIPCC, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True,
                        text=True).stdout.strip()
    if not os.path.isabs(rt) or not os.path.exists(rt):
        pytest.skip("no clang address-sanitizer runtime")
    from decode_step_token_sampler_amd import build as libbuild
    lib = str(tmp_path / "libdsts_sampler_san.so")
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-shared-libasan",
           "-Xarch_host", "-fno-omit-frame-pointer"]
    subprocess.check_call([HIPCC, *libbuild.FLAGS, *san, *libbuild.SOURCES, "-o", lib])
    _child({"LD_PRELOAD": rt, "DSTS_LIBRARY": lib}, ["tests/test_abi_cpu.py"], timeout=900)
