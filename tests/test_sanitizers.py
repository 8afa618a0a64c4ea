"""The oracle and the host-side argument checks under AddressSanitizer and
UndefinedBehaviorSanitizer (CPU only; host code, built with gcc/g++).

* The fp64 oracle (oracle/oracle.c) is built with -fsanitize=address,undefined
  and every oracle pin file runs against that build in a child process
  (the sanitizer runtimes preloaded, the build named by ORACLE_LIB): any
  out-of-bounds access, use after free, overflow or misaligned access aborts
  the child and fails the test.
* The library's host-side checks and work geometry (csrc/host_args.cpp)
  are built the same way with tests/host_args_check.cpp, which drives them
  through valid, invalid and extreme arguments.
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "speculative_decoding_rejection_spec_amd", "csrc")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]
ORACLE_PINS = ["test_oracle_pins.py", "test_oracle_flags.py", "test_oracle_draft.py", "test_oracle_rows.py",
               "test_oracle_bookkeeping.py", "test_oracle_golden.py"]

pytestmark = pytest.mark.skipif(shutil.which("gcc") is None or shutil.which("g++") is None,
                                reason="needs gcc and g++")


def _runtime(name):
    path = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True).stdout.strip()
    if not os.path.isabs(path) or not os.path.exists(path):
        pytest.skip(f"{name} not available")
    return path


@pytest.mark.slow
def test_oracle_pins_under_sanitizers(tmp_path):
    lib = str(tmp_path / "liboracle_san.so")
    subprocess.check_call(["gcc", "-std=c11", "-fPIC", "-shared", "-fno-fast-math", *SAN, "-o", lib,
                           os.path.join(ROOT, "oracle", "oracle.c"), "-lm"])
    env = dict(os.environ, ORACLE_LIB=lib,
               LD_PRELOAD=f"{_runtime('libasan.so')} {_runtime('libubsan.so')}",
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:xdist", "-p", "no:cacheprovider",
                        *[os.path.join(ROOT, "tests", f) for f in ORACLE_PINS]],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "runtime error" not in out and "AddressSanitizer" not in out, out[-4000:]


def test_host_argument_checks_under_sanitizers(tmp_path):
    exe = str(tmp_path / "host_args_check")
    subprocess.check_call(["g++", "-std=c++17", *SAN, "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
                           f"-I{CSRC}", os.path.join(CSRC, "host_args.cpp"),
                           os.path.join(ROOT, "tests", "host_args_check.cpp"), "-o", exe])
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300,
                       env=dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1"))
    assert r.returncode == 0 and r.stdout.strip() == "ok", (r.stdout + r.stderr)[-4000:]
