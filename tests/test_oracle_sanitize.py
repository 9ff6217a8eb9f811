"""The fp64 oracle under AddressSanitizer and UndefinedBehaviorSanitizer.

oracle/sdpa_f64.c is compiled together with tests/sanitize/oracle_driver.c
by gcc with -fsanitize=address,undefined (no recovery: the first report
aborts) and run on the CPU: heap overruns in the row loops, use after free
of the per-thread scratch, leaks, signed overflow in the index arithmetic
and the like fail the test.  Skipped if this gcc has no sanitizer runtime.
"""
import os
import shutil
import subprocess
from pathlib import Path

import pytest

ROOT = Path(__file__).resolve().parents[1]


def test_oracle_is_clean_under_asan_and_ubsan(tmp_path):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("no gcc")
    exe = tmp_path / "oracle_sanitized"
    cmd = [gcc, "-std=c11", "-g", "-O1", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", "-pthread", str(ROOT / "oracle" / "sdpa_f64.c"),
           str(ROOT / "tests" / "sanitize" / "oracle_driver.c"), "-o", str(exe), "-lm"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        if "asan" in r.stderr.lower() or "ubsan" in r.stderr.lower():
            pytest.skip(f"gcc has no sanitizer runtime: {r.stderr.strip()[:200]}")
        raise AssertionError(f"compile failed:\n{r.stderr}")
    # verify_asan_link_order=0: the run also works where the environment
    # preloads another library ahead of the sanitizer runtime
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:halt_on_error=1:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, f"sanitized oracle failed (rc {r.returncode}):\n{r.stdout}\n{r.stderr[-4000:]}"
    assert "all checks passed" in r.stdout


def test_the_sanitizer_build_catches_a_planted_overrun(tmp_path):
    """Negative control: a copy of the oracle whose probability loop writes
    one element past its row must fail under the same build and driver."""
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("no gcc")
    src = (ROOT / "oracle" / "sdpa_f64.c").read_text()
    good = "for (int64_t j = 0; j < jb->S; ++j) prow[j]"
    assert src.count(good) == 1
    bad = tmp_path / "sdpa_overrun.c"
    bad.write_text(src.replace(good, "for (int64_t j = 0; j <= jb->S; ++j) prow[j]"))
    exe = tmp_path / "oracle_overrun"
    cmd = [gcc, "-std=c11", "-g", "-O1", "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-pthread",
           str(bad), str(ROOT / "tests" / "sanitize" / "oracle_driver.c"), "-o", str(exe), "-lm"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        pytest.skip(f"no sanitizer build: {r.stderr.strip()[:200]}")
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:verify_asan_link_order=0")
    r = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode != 0 and "heap-buffer-overflow" in r.stderr
