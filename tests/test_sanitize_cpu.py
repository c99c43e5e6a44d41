"""CPU sanitizer run of the host code (AddressSanitizer + UndefinedBehavior-
Sanitizer, gcc/g++ only; no GPU code is built with a sanitizer):

- the oracle (oracle/bitlinear_oracle.c) built with the sanitizers and the
  whole pin suite (tests/test_oracle_pins.py) run against that build;
- the C ABI's argument validation (csrc/api.cpp with the host shape rules of
  csrc/shapes.cpp; the device launchers replaced by stubs that launch
  nothing) built with the sanitizers and the ABI rejection suite
  (tests/test_abi_cpu.py) run against it.

Each suite runs in a subprocess with the sanitizer runtimes preloaded (the
Python interpreter itself is not instrumented; leak checking is off because
of it).  Any sanitizer report aborts the subprocess, so the test fails."""

import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "bitlinear_rmsnorm_absmax_amd", "csrc")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]

pytestmark = pytest.mark.skipif(shutil.which("gcc") is None or shutil.which("g++") is None,
                                reason="needs gcc and g++")


def _runtime(name):
    return subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True,
                          check=True).stdout.strip()


def _env(extra):
    env = dict(os.environ)
    env.update(extra)
    env["LD_PRELOAD"] = f"{_runtime('libasan.so')}:{_runtime('libubsan.so')}"
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    env["PYTHONDONTWRITEBYTECODE"] = "1"
    return env


def _check(r):
    out = r.stdout[-4000:] + r.stderr[-4000:]
    assert "ERROR: AddressSanitizer" not in out and "runtime error:" not in out, out
    assert r.returncode == 0, out


def test_oracle_pins_under_sanitizers(tmp_path):
    lib = str(tmp_path / "liboracle_san.so")
    subprocess.run(["gcc", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fopenmp", "-fPIC",
                    "-shared", *SAN, "-o", lib, os.path.join(ROOT, "oracle", "bitlinear_oracle.c"),
                    "-lm"], check=True)
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                       capture_output=True, text=True, env=_env({"ORACLE_LIB": lib}), timeout=900,
                       cwd=ROOT)
    _check(r)


def test_abi_validation_under_sanitizers(tmp_path):
    lib = str(tmp_path / "libbitlinear_san.so")
    subprocess.run(["g++", "-std=c++17", "-fPIC", "-shared", *SAN, "-D__HIP_PLATFORM_AMD__",
                    "-I/opt/rocm/include", "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-o", lib,
                    os.path.join(CSRC, "api.cpp"), os.path.join(CSRC, "shapes.cpp"),
                    os.path.join(ROOT, "tests", "sanitize", "launch_stubs.cpp"),
                    "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib"], check=True)
    r = subprocess.run([sys.executable, os.path.join(ROOT, "tests", "sanitize", "run_abi_tests.py"),
                        lib], capture_output=True, text=True, env=_env({}), timeout=900, cwd=ROOT)
    _check(r)
