"""Inputs that drive the bf16 flash kernel's reference tracking, shared by
the GPU parity tests (which run them through the kernel) and the CPU tests
of a model of that tracking (which check that each case reaches the path it
is meant to exercise).  Test infrastructure only: no attention arithmetic of
the product lives here.

The kernel takes the exact row maximum of a query row's first 64-key tile
and starts the row's reference REF_MARGIN log2 units above it; later tiles
take no row maximum and instead check, per lane, the sum of their 32
probabilities 2^(x - m) against SPEC_LIMIT (x: score in log2 units).  A
failed check with finite probabilities is corrected in place; an infinite
probability (x - m >= 128) makes the whole query tile be recomputed
exactly.  Both constants restate the kernel's (kRefMargin, kSpecLimit).
"""
import numpy as np

from transformer_attention_micro_amd import inputs

REF_MARGIN = 64.0
SPEC_LIMIT = 4096.0


def growing_keys(d, causal, jump, S=1024, H=2):
    """Keys scaled by powers of two (exact in bf16) along the key axis: in
    steps (x2 per 128 keys up to x16), or at once (x256 from key 320 on)."""
    p = inputs.make_problem(1, H, S, d, inputs.BF16, causal=causal, seed=11)
    j = np.arange(p.S)
    if jump:
        f = np.where(j >= 320, 256.0, 1.0)
    else:
        f = 2.0 ** np.minimum(j // 128, 4)
    p.k[:] = (p.k * f[None, :, None]).astype(np.float32)
    return p


def diagonal_keys(d, scale, H=128, S=1024):
    """Causal; keys from 448 on scaled by `scale` (a power of two).  Key tile
    7 (keys 448..511) is the diagonal tile of the waves at rows 448..511."""
    p = inputs.make_problem(1, H, S, d, inputs.BF16, causal=True, seed=13)
    f = np.where(np.arange(p.S) >= 448, scale, 1.0)
    p.k[:] = (p.k * f[None, :, None]).astype(np.float32)
    return p


# Every query is 32 e_0; keys 0..63 have a zero first coordinate (scores 0,
# so the reference is REF_MARGIN), the others `a`: bf16-exact values with
# 32 a log2(e) / sqrt(d) - REF_MARGIN = 126.4 .. 127.8, so every later
# probability is finite in bf16 and fp32 while a lane's sum of 32 of them
# overflows fp32.
SUM_OVERFLOW_A = {32: 23.5, 64: 33.0, 128: 47.0}


def sum_overflow_problem(d, causal):
    p = inputs.make_problem(1, 2, 512, d, inputs.BF16, causal=causal, seed=12)
    p.q[:] = 0.0
    p.q[:, :, 0] = 32.0
    p.k[:, :64, 0] = 0.0
    p.k[:, 64:, 0] = SUM_OVERFLOW_A[d]
    return p


def sum_overflow_log2_score(d):
    """The later keys' score in log2 units above the reference."""
    return 32.0 * SUM_OVERFLOW_A[d] * np.log2(np.e) / np.sqrt(d) - REF_MARGIN


def first_tile_dominant(d, causal, scale=64.0, S=600, H=3):
    """Keys 0..63 scaled by `scale` (a power of two): the first tile's row
    maximum sits well over a hundred log2 units above every later score, so
    with the margin every later probability falls below the fp32 normal
    range and underflows; their weight is negligible in the exact result
    too."""
    p = inputs.make_problem(1, H, S, d, inputs.BF16, causal=causal, seed=14)
    f = np.where(np.arange(p.S) < 64, scale, 1.0)
    p.k[:] = (p.k * f[None, :, None]).astype(np.float32)
    return p
