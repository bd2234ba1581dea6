"""The oracle's C source built with AddressSanitizer and UndefinedBehavior-
Sanitizer (gcc, host code only), with the CPU pins and the randomised
property tests run against that build in a child process (the sanitizer
runtime preloaded, since the Python interpreter itself is not instrumented).

A negative control plants an out-of-bounds read in a copy of the source and
requires the sanitizer to stop the run with a heap-buffer-overflow report,
so a silently inactive sanitizer cannot pass."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "selscan_ref.c")
CFLAGS = ["-O1", "-g", "-std=c99", "-fno-fast-math", "-ffp-contract=off", "-fPIC", "-shared",
          "-pthread", "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
          "-fno-omit-frame-pointer"]


def _runtime(name):
    path = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True,
                          text=True).stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


ASAN, UBSAN = _runtime("libasan.so"), _runtime("libubsan.so")
pytestmark = pytest.mark.skipif(not (ASAN and UBSAN), reason="gcc sanitizer runtimes not found")


def _build(src, out):
    subprocess.run(["gcc", *CFLAGS, src, "-o", out, "-lm"], check=True)


def _run_under_sanitizers(lib, tests, extra=()):
    env = dict(os.environ)
    env.update(SELSCAN_ORACLE_LIB=lib, LD_PRELOAD=f"{ASAN} {UBSAN}",
               ASAN_OPTIONS="detect_leaks=0:verify_asan_link_order=0:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    # -s: a sanitizer report is written to fd 2 and the process ends; with
    # pytest capturing fd 2 the report would be lost.
    cmd = [sys.executable, "-m", "pytest", "-q", "-s", "-x", "-p", "no:cacheprovider",
           "-p", "no:xdist", *tests, *extra]
    return subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)


def test_pins_and_properties_clean_under_asan_ubsan(tmp_path):
    lib = str(tmp_path / "libselscan_ref_san.so")
    _build(SRC, lib)
    res = _run_under_sanitizers(lib, ["tests/test_oracle_pins.py", "tests/test_oracle_props.py"])
    out = res.stdout + res.stderr
    assert res.returncode == 0, out[-4000:]
    assert "ERROR: AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]


def test_planted_out_of_bounds_read_is_reported(tmp_path):
    with open(SRC) as f:
        text = f.read()
    needle = "acc += Cb[n * L + t] * h[n];"
    assert text.count(needle) == 1
    bad = tmp_path / "selscan_ref_oob.c"
    bad.write_text(text.replace(needle, "acc += Cb[n * L + t + 1] * h[n];"))
    lib = str(tmp_path / "libselscan_ref_oob.so")
    _build(str(bad), lib)
    res = _run_under_sanitizers(lib, ["tests/test_oracle_pins.py"], ["-k", "run_ssm_printed or lti_convolution_direct"])
    out = res.stdout + res.stderr
    assert res.returncode != 0
    assert "heap-buffer-overflow" in out, out[-4000:]
