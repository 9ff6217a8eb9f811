"""Seeded synthetic inputs for the attention forward pass.

This module is shared by the GPU path's tests and benchmark and by the oracle's
tests.  It holds none of the attention arithmetic: it draws i.i.d. N(0, 1)
values, rounds them to the input dtype and lays them out as [B*H, S, d]
row-major (the flattened batch*heads layout of the kbench page, section
"The three GPU kernels").

Recipe, for a problem (B, H, S, d, dtype, seed):
  1. ``numpy.random.default_rng(seed).standard_normal`` draws B*H*S*d float64
     values for Q, then for K, then for V, from one stream.
  2. Each value is rounded to float32 (round to nearest even).
  3. bf16 problems round the float32 value once more to bfloat16 (round to
     nearest even, ties to even) on the host.  Both sides consume exactly
     these values: the GPU as bf16 bits, the oracle as the same numbers
     widened to float32.
  4. An optional power-of-two ``q_scale`` (the large-logit stability case
     multiplies the bf16 Q by 8) is applied after rounding, which is exact.
"""
from __future__ import annotations

import hashlib
from dataclasses import dataclass

import numpy as np

F32 = "f32"
BF16 = "bf16"


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16, round-to-nearest-even; returns the
    16-bit patterns as uint16.  NaN stays NaN (quietened), +-Inf stays Inf,
    values that round past the largest finite bf16 become Inf."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    is_nan = (u & np.uint32(0x7FFFFFFF)) > np.uint32(0x7F800000)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)
    if is_nan.any():
        r[is_nan] = ((u[is_nan] >> np.uint32(16)) | np.uint32(0x0040)).astype(np.uint16)
    return r


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bit patterns to the float32 values they denote (exact)."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclass
class Problem:
    """One attention problem: sizes, dtype and the exact input values."""
    B: int
    H: int
    S: int
    d: int
    dtype: str
    causal: bool
    q: np.ndarray  # float32 [B*H, S, d], exact input values
    k: np.ndarray
    v: np.ndarray
    seed: int
    q_scale: float = 1.0

    @property
    def BH(self) -> int:
        return self.B * self.H

    def device_arrays(self):
        """The arrays handed to the GPU: float32 as is, bf16 as uint16 bits."""
        if self.dtype == F32:
            return self.q, self.k, self.v
        return bf16_bits(self.q), bf16_bits(self.k), bf16_bits(self.v)

    def sha256(self) -> str:
        h = hashlib.sha256()
        for a in self.device_arrays():
            h.update(np.ascontiguousarray(a).tobytes())
        return h.hexdigest()


def make_problem(B: int, H: int, S: int, d: int, dtype: str = F32, causal: bool = False,
                 seed: int = 0, q_scale: float = 1.0) -> Problem:
    """Draw Q, K, V per the recipe in the module docstring."""
    if dtype not in (F32, BF16):
        raise ValueError(f"dtype must be {F32!r} or {BF16!r}")
    if q_scale <= 0 or np.log2(q_scale) != int(np.log2(q_scale)):
        raise ValueError("q_scale must be a power of two (so scaling stays exact)")
    n = B * H * S * d
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(3):
        x = rng.standard_normal(n, dtype=np.float64).astype(np.float32)
        if dtype == BF16:
            x = bf16_bits_to_f32(bf16_bits(x))
        out.append(x.reshape(B * H, S, d))
    q, k, v = out
    if q_scale != 1.0:
        q = (q * np.float32(q_scale)).astype(np.float32)
    return Problem(B, H, S, d, dtype, bool(causal), q, k, v, seed, q_scale)


# The workloads the measurements are quoted on (sizes from the task's problem
# list; names say what they are).
WORKLOADS = {
    "b1h1s64d32_f32": dict(B=1, H=1, S=64, d=32, dtype=F32, causal=False),
    "b1h8s512d64_f32": dict(B=1, H=8, S=512, d=64, dtype=F32, causal=False),
    "b1h8s512d64_f32_causal": dict(B=1, H=8, S=512, d=64, dtype=F32, causal=True),
    "b4h16s2048d64_bf16_causal": dict(B=4, H=16, S=2048, d=64, dtype=BF16, causal=True),
    "b2h32s8192d128_bf16_causal": dict(B=2, H=32, S=8192, d=128, dtype=BF16, causal=True),
    "b2h32s8192d128_bf16_causal_q8": dict(B=2, H=32, S=8192, d=128, dtype=BF16, causal=True,
                                          q_scale=8.0),
    "b1h16s32768d128_bf16": dict(B=1, H=16, S=32768, d=128, dtype=BF16, causal=False),
}


def workload(name: str, seed: int = 0) -> Problem:
    return make_problem(seed=seed, **WORKLOADS[name])

