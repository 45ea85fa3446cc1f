"""The CPU tier under AddressSanitizer (and UBSan for the oracle): the C-ABI
host layer (kda_api.cpp: every argument check, workspace sizing, failure
injection) and the C oracle are rebuilt with -fsanitize, and the CPU tests
that exercise them run again in a child process with the sanitizer runtime
preloaded. Any sanitizer report fails the test. CPU only: the GPU launchers
are replaced by host stubs that report no device (tests/asan/launch_stub.cpp).
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "linear_attention_recurrence_11_amd", "csrc")
HERE = os.path.join(ROOT, "tests", "asan")
SAN = ["-fsanitize=address", "-fno-omit-frame-pointer", "-g", "-O1"]
# the CPU tests that reach the C-ABI layer or the C oracle
CHILD_TESTS = ["tests/test_abi.py", "tests/test_binding_checks.py", "tests/test_oracle_pins.py",
               "tests/test_oracle_gate.py", "tests/test_oracle_mutants.py"]


def _libasan():
    path = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True,
                          text=True).stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


@pytest.fixture(scope="module")
def asan_libs(tmp_path_factory):
    if not shutil.which("gcc") or not shutil.which("g++") or not _libasan():
        pytest.skip("gcc with AddressSanitizer is not available")
    out = tmp_path_factory.mktemp("asan")
    host = str(out / "libkda_host_asan.so")
    orc = str(out / "libkda_oracle_asan.so")
    subprocess.run(["g++", "-std=c++17", "-shared", "-fPIC", *SAN, "-D__HIP_PLATFORM_AMD__",
                    "-I/opt/rocm/include", "-I" + os.path.join(ROOT, "include"), "-I" + CSRC,
                    os.path.join(CSRC, "kda_api.cpp"), os.path.join(HERE, "launch_stub.cpp"),
                    "-o", host], check=True)
    subprocess.run(["gcc", "-shared", "-fPIC", "-pthread", *SAN, "-fsanitize=undefined",
                    "-fno-sanitize-recover=undefined",
                    os.path.join(ROOT, "oracle", "kda_oracle.c"), "-o", orc, "-lm"], check=True)
    return host, orc


def test_cpu_tier_under_address_sanitizer(asan_libs):
    host, orc = asan_libs
    env = dict(os.environ)
    env.update(LD_PRELOAD=_libasan(), ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1",
               KDA_ASAN_HOST_LIB=host, KDA_ASAN_ORACLE_LIB=orc,
               PYTHONPATH=os.pathsep.join([ROOT, HERE, env.get("PYTHONPATH", "")]))
    res = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-m", "not gpu",
                          "-p", "asan_plugin", "-p", "no:cacheprovider",
                          # reports go to the process stderr, not into a capture file
                          "--capture=sys", *CHILD_TESTS],
                         cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    out = res.stdout + res.stderr
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert res.returncode == 0, out[-4000:]
    assert " passed" in out
