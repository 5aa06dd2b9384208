"""The oracle's host code under the address and undefined-behaviour sanitizers
(CPU only): oracle/sanitize_driver.c calls every oracle entry point over every
descriptor combination, with finite inputs and then with NaN and infinities.
The sanitized build must run clean, and its results on finite inputs must
equal a plain optimized build's bit for bit."""
import os
import re
import subprocess

import pytest

import oracle

HERE = os.path.dirname(oracle.__file__)
SOURCES = [os.path.join(HERE, "sanitize_driver.c"), os.path.join(HERE, "lq_oracle.c")]
COMMON = ["-std=c11", "-ffp-contract=off", "-fno-fast-math", "-I", HERE]
# float-cast-overflow is not part of GCC's -fsanitize=undefined; it catches a
# NaN or out-of-range value converted to an integer
SANITIZE = ["-O1", "-g", "-fsanitize=address,undefined,float-cast-overflow", "-fno-sanitize-recover=all",
            "-fno-omit-frame-pointer"]


def _build_and_run(tmp_path, name, flags):
    exe = str(tmp_path / name)
    subprocess.run(["gcc", *COMMON, *flags, *SOURCES, "-o", exe, "-lm"], check=True, capture_output=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    return r


def test_oracle_clean_under_sanitizers(tmp_path):
    san = _build_and_run(tmp_path, "sanitized", SANITIZE)
    assert san.returncode == 0, san.stderr[-4000:]
    assert "runtime error" not in san.stderr and "Sanitizer" not in san.stderr, san.stderr[-4000:]
    plain = _build_and_run(tmp_path, "plain", ["-O2"])
    assert plain.returncode == 0, plain.stderr[-2000:]
    pat = r"digest ([0-9a-f]{16}) nonfinite ([0-9a-f]{16}) calls (\d+)"
    a, b = re.search(pat, san.stdout), re.search(pat, plain.stdout)
    assert a and b, (san.stdout, plain.stdout)
    assert a.group(1) == b.group(1), "results on finite inputs differ between the sanitized and plain builds"
    assert a.group(3) == b.group(3) and int(a.group(3)) > 10000
