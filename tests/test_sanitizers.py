"""CPU: the host-side code under address and undefined-behaviour sanitizers.

1. libmoe's host rules (combine_topk_ids_amd/csrc/host_checks.cpp: every
   argument check, size and launch-geometry rule of the C ABI) are built with
   g++ -fsanitize=address,undefined together with the fuzz driver
   tests/sanitize/host_checks_fuzz.cpp and run over two million random
   problems (edge values of every field, null, aligned and misaligned
   pointers); any sanitizer report or broken guarantee fails the test.
2. The oracle (oracle/oracle.c) is built the same way and the oracle's pin
   tests run against that build (ORACLE_PREBUILT_LIB, with the sanitizer
   runtimes preloaded into the Python process), so every buffer the Python
   side hands to the C loops is checked for overruns.
No GPU is used.
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g",
       "-O1"]

pytestmark = pytest.mark.skipif(shutil.which("g++") is None or shutil.which("gcc") is None,
                                reason="needs gcc and g++")


def _runtime(name):
    path = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True,
                          check=True).stdout.strip()
    if not os.path.isabs(path) or not os.path.exists(path):
        pytest.skip(f"{name} not found")
    return path


def test_host_checks_under_sanitizers(tmp_path):
    exe = str(tmp_path / "host_checks_fuzz")
    subprocess.run(["g++", "-std=c++17", "-Wall"] + SAN +
                   ["-I", os.path.join(ROOT, "include"),
                    "-I", os.path.join(ROOT, "combine_topk_ids_amd", "csrc"),
                    os.path.join(ROOT, "combine_topk_ids_amd", "csrc", "host_checks.cpp"),
                    os.path.join(ROOT, "tests", "sanitize", "host_checks_fuzz.cpp"), "-o", exe],
                   check=True)
    res = subprocess.run([exe, "2000000"], capture_output=True, text=True, timeout=300,
                         env={**os.environ, "ASAN_OPTIONS": "detect_leaks=1:abort_on_error=0",
                              "UBSAN_OPTIONS": "print_stacktrace=1"})
    assert res.returncode == 0, res.stdout + res.stderr
    assert "runtime error" not in res.stderr and "AddressSanitizer" not in res.stderr
    assert "no failures" in res.stdout


def test_oracle_pins_under_sanitizers(tmp_path):
    lib = str(tmp_path / "liboracle_sanitized.so")
    subprocess.run(["gcc", "-std=c99", "-fPIC", "-shared", "-ffp-contract=off", "-fopenmp",
                    "-Wall"] + SAN + ["-o", lib, os.path.join(ROOT, "oracle", "oracle.c"), "-lm"],
                   check=True)
    pins = sorted(os.path.join(ROOT, "tests", f) for f in os.listdir(os.path.join(ROOT, "tests"))
                  if f.startswith("test_oracle_") and f.endswith(".py"))
    env = {**os.environ, "ORACLE_PREBUILT_LIB": lib,
           "LD_PRELOAD": _runtime("libasan.so") + ":" + _runtime("libubsan.so"),
           "ASAN_OPTIONS": "detect_leaks=0", "UBSAN_OPTIONS": "print_stacktrace=1",
           "OMP_NUM_THREADS": "4"}
    res = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider"] + pins,
                         cwd=ROOT, capture_output=True, text=True, timeout=900, env=env)
    out = res.stdout + res.stderr
    assert res.returncode == 0, out[-4000:]
    assert "runtime error" not in out and "AddressSanitizer" not in out
