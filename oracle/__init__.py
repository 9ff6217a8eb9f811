"""fp64 CPU oracle for the scaled dot-product attention forward pass.

TEST INFRASTRUCTURE ONLY.  This package is the checker the GPU kernels are
compared against.  Only the test suite, the smoke check and the benchmark's
CPU-baseline leg may import it; the product library never does, and it shares
no code, header or constant with the GPU path.

The arithmetic lives in ``sdpa_f64.c`` (plain C, double precision, libm exp),
which follows the definition on the kbench page, section "The three GPU
kernels": O = softmax(Q K^T / sqrt(d)) V over a flattened batch*heads axis in
[head, seq, dim] row-major layout, with the causal reading "key j visible to
query i iff j <= i".  This module only builds the shared object, marshals
numpy arrays and picks the thread count.

Pins (tests/test_oracle_*.py): brute force in 50-digit decimal arithmetic on
tiny shapes, closed forms (two keys; uniform weights; hardmax limit; rational
golden cases), and the invariants softmax rows sum to one, identical value
rows reproduce that row, Q = 0 gives the (prefix) mean of V, permuting K/V
rows together changes nothing without a mask, and a common shift of all keys
changes nothing.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import sys
from pathlib import Path

import numpy as np

_HERE = Path(__file__).resolve().parent
_SRC = _HERE / "sdpa_f64.c"
_LIB = _HERE / "libkb_oracle.so"
_handle = None


def build(force: bool = True) -> Path:
    """Compile sdpa_f64.c with gcc (no fast-math: libm exp, IEEE double)."""
    if force or not _LIB.exists() or _LIB.stat().st_mtime < _SRC.stat().st_mtime:
        tmp = _LIB.with_suffix(".so.tmp")
        cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread",
               str(_SRC), "-o", str(tmp), "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _lib():
    global _handle
    if _handle is None:
        if not _LIB.exists() or _LIB.stat().st_mtime < _SRC.stat().st_mtime:
            build(force=True)
        h = ctypes.CDLL(str(_LIB))
        argt = [ctypes.c_void_p] * 3 + [ctypes.c_int64] * 3 + [ctypes.c_int, ctypes.c_double,
                                                              ctypes.c_void_p, ctypes.c_int64,
                                                              ctypes.c_void_p, ctypes.c_int]
        for name in ("kbo_sdpa_rows", "kbo_probs_rows"):
            fn = getattr(h, name)
            fn.argtypes = argt
            fn.restype = ctypes.c_int
        _handle = h
    return _handle


def default_threads() -> int:
    """Threads the oracle uses by default: the CPUs this process may run on."""
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover - non-Linux
        return max(1, os.cpu_count() or 1)


def _prep(Q, K, V):
    Q = np.ascontiguousarray(Q, dtype=np.float32)
    K = np.ascontiguousarray(K, dtype=np.float32)
    V = np.ascontiguousarray(V, dtype=np.float32)
    if Q.ndim != 3 or Q.shape != K.shape or Q.shape != V.shape:
        raise ValueError(f"Q, K, V must share one [BH, S, d] shape, got {Q.shape}, {K.shape}, {V.shape}")
    return Q, K, V


def _rows(rows, BH, S):
    if rows is None:
        return None, BH * S
    r = np.ascontiguousarray(rows, dtype=np.int64).reshape(-1)
    if r.size and (r.min() < 0 or r.max() >= BH * S):
        raise ValueError("row id out of range")
    return r, r.size


def sdpa(Q, K, V, causal: bool = False, scale: float | None = None, rows=None,
         nthreads: int | None = None) -> np.ndarray:
    """fp64 attention output.

    Q, K, V: float32-representable arrays of shape [BH, S, d].  ``rows`` is an
    optional array of flat row ids ``bh * S + i``; without it every row is
    computed and the result has shape [BH, S, d], with it the result has shape
    [len(rows), d].  ``scale`` defaults to 1/sqrt(d).
    """
    Q, K, V = _prep(Q, K, V)
    BH, S, d = Q.shape
    r, n = _rows(rows, BH, S)
    out = np.empty((n, d), dtype=np.float64)
    if n == 0:
        return out
    nt = nthreads or default_threads()
    rc = _lib().kbo_sdpa_rows(Q.ctypes.data, K.ctypes.data, V.ctypes.data, BH, S, d,
                              int(bool(causal)), float(scale or 0.0),
                              None if r is None else r.ctypes.data, n,
                              out.ctypes.data, int(nt))
    if rc != 0:
        raise RuntimeError(f"oracle kbo_sdpa_rows failed with status {rc}")
    return out.reshape(BH, S, d) if r is None else out


def probs(Q, K, V, causal: bool = False, scale: float | None = None, rows=None,
          nthreads: int | None = None) -> np.ndarray:
    """fp64 softmax probabilities P[i, j] (masked keys exactly 0).

    Shape [BH, S, S] without ``rows``, [len(rows), S] with it.
    """
    Q, K, V = _prep(Q, K, V)
    BH, S, d = Q.shape
    r, n = _rows(rows, BH, S)
    out = np.empty((n, S), dtype=np.float64)
    if n == 0:
        return out
    nt = nthreads or default_threads()
    rc = _lib().kbo_probs_rows(Q.ctypes.data, K.ctypes.data, V.ctypes.data, BH, S, d,
                               int(bool(causal)), float(scale or 0.0),
                               None if r is None else r.ctypes.data, n,
                               out.ctypes.data, int(nt))
    if rc != 0:
        raise RuntimeError(f"oracle kbo_probs_rows failed with status {rc}")
    return out.reshape(BH, S, S) if r is None else out


if __name__ == "__main__":  # pragma: no cover
    build(force=True)
    print(f"built {_LIB}", file=sys.stderr)
