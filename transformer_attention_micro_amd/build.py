"""Build libkb.so (the gfx950 HIP kernels and their C ABI) in-tree.

    python -m transformer_attention_micro_amd.build

Every .hip file under csrc/ is compiled for gfx950 only, position
independent, then linked into transformer_attention_micro_amd/libkb.so.
Packed fp32 instructions are disabled for all device code.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor
from pathlib import Path

PKG = Path(__file__).resolve().parent
ROOT = PKG.parent
CSRC = PKG / "csrc"
INCLUDE = ROOT / "include"
BUILD_DIR = ROOT / "_build"
LIB = PKG / "libkb.so"
ARCH = "gfx950"

HIPCC_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-command-line-argument", "-Wno-unknown-warning-option",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


# Extra flags per source.  The flash kernel takes row maxima of MFMA results;
# without relaxed NaN handling every fmaxf input is first canonicalised (one
# extra VALU op per score).  Its inputs are finite or -inf, never NaN.
FILE_FLAGS = {"attn_flash.hip": ["-fno-honor-nans", "-mllvm", "-amdgpu-mfma-vgpr-form"]}


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and Path(cand).exists():
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libkb.so)")


def sources() -> list[Path]:
    return sorted(CSRC.glob("*.hip"))


def _compile(src: Path) -> Path:
    obj = BUILD_DIR / (src.stem + ".o")
    cmd = [hipcc(), "-c", *HIPCC_FLAGS, *FILE_FLAGS.get(src.name, []), str(src), "-o", str(obj)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compiling {src.name} failed:\n{r.stderr}")
    return obj


def build(verbose: bool = False) -> Path:
    """Compile every kernel source and link libkb.so; returns its path."""
    BUILD_DIR.mkdir(exist_ok=True)
    srcs = sources()
    if not srcs:
        raise RuntimeError(f"no .hip sources under {CSRC}")
    jobs = max(1, min(len(srcs), int(os.environ.get("MAX_JOBS", "8"))))
    with ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB.with_name(LIB.name + ".tmp")
    cmd = [hipcc(), "-shared", f"--offload-arch={ARCH}", *map(str, objs), "-o", str(tmp)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"linking libkb.so failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB} from {len(srcs)} sources", file=sys.stderr)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
