"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

csrc/abi.hip (argument validation, size and overlap arithmetic, the timing
loop, error strings, the per-thread last error) is compiled with hipcc with
both sanitizers on its host code (no recovery: the first report aborts) and
linked with the kernel objects of the regular build into a driver,
tests/sanitize/abi_driver.c, that calls every entry point with arguments the
library must reject, or, without a GPU, stop at the device query; nothing is
launched.  A planted 32-bit overflow in a copy of abi.hip must be caught.
Skipped when the regular build's kernel objects or the sanitizer runtime are
missing.
"""
import os
import shutil
import subprocess
from pathlib import Path

import pytest

ROOT = Path(__file__).resolve().parents[1]
CSRC = ROOT / "transformer_attention_micro_amd" / "csrc"
BUILD = ROOT / "_build"
KERNELS = ("attn_flash", "attn_naive", "attn_fused", "triad", "ceiling")
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
CLANG = "/opt/rocm/llvm/bin/clang"
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:halt_on_error=1:verify_asan_link_order=0",
           UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")


def _build(tmp_path, abi_src):
    objs = [BUILD / f"{k}.o" for k in KERNELS]
    if not Path(HIPCC).exists() or not Path(CLANG).exists() or not all(o.exists() for o in objs):
        pytest.skip("needs hipcc, ROCm's clang and the regular build's kernel objects (_build/*.o)")
    base = ["-O1", "-g", "-std=c++17", "-fPIC", "--offload-arch=gfx950", "-fno-omit-frame-pointer",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", f"-I{ROOT / 'include'}", f"-I{CSRC}"]
    san = ["-Xarch_host", "-fsanitize=address",
           "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all"]
    abi_o, drv_o, exe = tmp_path / "abi.o", tmp_path / "driver.o", tmp_path / "abi_sanitized"
    steps = [
        [HIPCC, "-c", *base, *san, str(abi_src), "-o", str(abi_o)],
        [CLANG, "-c", "-std=c11", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
         "-fno-sanitize-recover=all", f"-I{ROOT / 'include'}", str(ROOT / "tests" / "sanitize" / "abi_driver.c"),
         "-o", str(drv_o)],
        [HIPCC, "--offload-arch=gfx950", "-Xarch_host", "-fsanitize=address",
         "-Xarch_host", "-fsanitize=undefined", str(drv_o), str(abi_o), *map(str, objs), "-o", str(exe),
         "-lpthread"],
    ]
    for cmd in steps:
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            if "asan" in r.stderr.lower() or "sanitizer" in r.stderr.lower():
                pytest.skip(f"no sanitizer runtime: {r.stderr.strip()[:200]}")
            raise AssertionError(f"build failed: {' '.join(cmd[:3])} ...\n{r.stderr[-3000:]}")
    return exe


def test_host_code_is_clean_under_asan_and_ubsan(tmp_path):
    exe = _build(tmp_path, CSRC / "abi.hip")
    r = subprocess.run([str(exe)], capture_output=True, text=True, env=ENV, timeout=300)
    assert r.returncode == 0, f"sanitized host code failed (rc {r.returncode}):\n{r.stdout}\n{r.stderr[-4000:]}"
    assert "all checks passed" in r.stdout


def test_the_sanitizer_build_catches_a_planted_overflow(tmp_path):
    """Negative control: the slice count multiplied in 32-bit int (65536 x
    65536 overflows) must stop the same build and driver."""
    src = (CSRC / "abi.hip").read_text()
    good = "const long long bh = (long long)cfg->batch * cfg->heads;"
    assert src.count(good) == 1
    bad = tmp_path / "abi_overflow.hip"
    bad.write_text(src.replace(good, "const long long bh = cfg->batch * cfg->heads;"))
    exe = _build(tmp_path, bad)
    r = subprocess.run([str(exe)], capture_output=True, text=True, env=ENV, timeout=300)
    assert r.returncode != 0 and "signed integer overflow" in r.stderr, r.stderr[-2000:]
