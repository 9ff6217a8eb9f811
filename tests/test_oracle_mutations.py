"""The oracle's pins must catch plausible mistakes (CPU only).

Each case compiles a copy of oracle/sdpa_f64.c with one planted mistake (a
dropped term, a wrong index or stride, an off-by-one in the mask, a flipped
comparison), swaps it in for the real oracle, and runs every pin in
tests/test_oracle.py.  At least one pin has to fail for every mutant.  The
mistakes are planted in the oracle, on the CPU, and never reach the GPU.
"""
import ctypes
import inspect
import os
import subprocess

import pytest

import oracle
from tests import test_oracle as pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "sdpa_f64.c")

MUTANTS = {
    "scale_dropped": ("s[j] = scale * dot;", "s[j] = dot;"),
    "causal_off_by_one": ("return causal ? i + 1 : S;", "return causal ? (i + 2 < S ? i + 2 : S) : S;"),
    "key_index_transposed": ("(double)Kh[j * d + k]", "(double)Kh[(k * nvis + j) % (nvis * d)]"),
    "value_row_shifted": ("(double)Vh[j * d + k]", "(double)Vh[((j + 1) % nvis) * d + k]"),
    "head_stride_wrong": ("const float *Kh = jb->K + bh * jb->S * jb->d;",
                          "const float *Kh = jb->K + (bh > 0 ? bh - 1 : 0) * jb->S * jb->d;"),
    "no_max_subtraction": ("s[j] = exp(s[j] - m);", "s[j] = exp(s[j]);"),
    "min_instead_of_max": ("if (s[j] > m) m = s[j];", "if (s[j] < m) m = s[j];"),
    "normalisation_dropped": ("for (int64_t k = 0; k < d; ++k) o[k] /= Z;", ""),
    "query_row_shifted": ("jb->Q + (bh * jb->S + i) * jb->d", "jb->Q + (bh * jb->S + (i + 1) % jb->S) * jb->d"),
}


def _pin_functions():
    out = []
    for name, fn in inspect.getmembers(pins, inspect.isfunction):
        if not name.startswith("test_") or name == "test_rejects_bad_arguments":
            continue
        marks = getattr(fn, "pytestmark", [])
        params = [m for m in marks if m.name == "parametrize"]
        combos = [{}]
        for m in params:
            argnames = [a.strip() for a in (m.args[0].split(",") if isinstance(m.args[0], str) else m.args[0])]
            new = []
            for c in combos:
                for val in m.args[1]:
                    vals = val if len(argnames) > 1 else (val,)
                    new.append({**c, **dict(zip(argnames, vals))})
            combos = new
        for c in combos:
            out.append((name, fn, c))
    return out


@pytest.mark.parametrize("mutant", sorted(MUTANTS))
def test_pins_catch_mutant(mutant, tmp_path):
    before, after = MUTANTS[mutant]
    src = open(SRC).read()
    assert src.count(before) == 1, f"mutation anchor for {mutant} not found exactly once"
    mutated = tmp_path / "mut.c"
    mutated.write_text(src.replace(before, after))
    so = tmp_path / "libmut.so"
    subprocess.run(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread", str(mutated), "-o", str(so), "-lm"],
                   check=True)
    real = oracle._lib()
    h = ctypes.CDLL(str(so))
    for n in ("kbo_sdpa_rows", "kbo_probs_rows"):
        getattr(h, n).argtypes = getattr(real, n).argtypes
        getattr(h, n).restype = ctypes.c_int
    caught = []
    oracle._handle = h
    try:
        for name, fn, kwargs in _pin_functions():
            try:
                fn(**kwargs)
            except Exception:  # AssertionError, or a NaN/overflow error
                caught.append(name)
    finally:
        oracle._handle = real
    assert caught, f"no pin caught mutant {mutant}"
