"""AddressSanitizer and UndefinedBehaviorSanitizer builds of the host code, on
the CPU: the plain-C oracle (oracle/skip_attention_c.c) and the host
configuration functions (csrc/ssa_config.cpp), each linked with a driver
under tests/sanitize/ that runs every entry point, argument errors and
ragged shapes included.  Host code only, built with gcc / g++; no GPU code is
built with a sanitizer.  A sanitizer report aborts the driver, which fails
the test."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]
ENV = {**os.environ, "ASAN_OPTIONS": "detect_leaks=1:abort_on_error=1",
       "UBSAN_OPTIONS": "print_stacktrace=1:halt_on_error=1", "OMP_NUM_THREADS": "4"}


def _build_and_run(tmp_path, compiler, sources, extra):
    if shutil.which(compiler) is None:
        pytest.skip(f"{compiler} not available")
    exe = str(tmp_path / "driver")
    r = subprocess.run([compiler, *SAN, *extra, "-o", exe, *sources, "-lm"], capture_output=True, text=True,
                       timeout=300)
    assert r.returncode == 0, r.stderr[-3000:]
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=ENV)
    out = r.stdout + r.stderr
    assert r.returncode == 0 and "ERROR: AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    return out


def test_oracle_under_asan_ubsan(tmp_path):
    out = _build_and_run(tmp_path, "gcc", [os.path.join(ROOT, "oracle", "skip_attention_c.c"),
                                           os.path.join(HERE, "oracle_driver.c")],
                         ["-std=c99", "-ffp-contract=off", "-fopenmp"])
    assert "0 failures" in out


def test_config_under_asan_ubsan(tmp_path):
    out = _build_and_run(tmp_path, "g++", [os.path.join(ROOT, "skip_softmax_flashattention_amd", "csrc",
                                                        "ssa_config.cpp"),
                                           os.path.join(HERE, "config_driver.cpp")],
                         ["-std=c++17", "-I" + os.path.join(ROOT, "include")])
    assert "0 failures" in out
