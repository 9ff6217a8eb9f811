"""Seeded input generator: determinism and bfloat16 rounding (CPU only).

bf16 rounding is checked against hand-picked bit patterns whose correct
round-to-nearest-even result follows from the format definition (8 exponent
bits, 7 stored mantissa bits), not against another implementation.
"""
import numpy as np
import pytest

from transformer_attention_micro_amd import inputs


def _f(bits):
    return np.array(bits, dtype=np.uint32).view(np.float32)


def test_bf16_round_to_nearest_even_cases():
    cases = [
        (0x3F800000, 0x3F80),  # 1.0 exact
        (0x3F808000, 0x3F80),  # halfway, lower neighbour even -> stays
        (0x3F818000, 0x3F82),  # halfway, lower neighbour odd -> rounds up
        (0x3F808001, 0x3F81),  # just above halfway -> up
        (0x3F807FFF, 0x3F80),  # just below halfway -> down
        (0x80000000, 0x8000),  # -0
        (0x00000001, 0x0000),  # smallest subnormal rounds to +0
        (0x00008000, 0x0000),  # halfway subnormal, even -> 0
        (0x00018000, 0x0002),  # halfway subnormal, odd -> up
        (0x7F800000, 0x7F80),  # +inf
        (0xFF800000, 0xFF80),  # -inf
        (0x7F7FFFFF, 0x7F80),  # max finite fp32 rounds past max bf16 -> inf
        (0x7F7F7FFF, 0x7F7F),  # just below the overflow threshold
    ]
    src = _f([c[0] for c in cases])
    got = inputs.bf16_bits(src)
    assert [int(g) for g in got] == [c[1] for c in cases]
    nan = inputs.bf16_bits(_f([0x7FC00001, 0x7F800001]))
    assert all((int(n) & 0x7F80) == 0x7F80 and (int(n) & 0x7F) != 0 for n in nan)


def test_bf16_widen_is_exact_and_idempotent():
    x = np.random.default_rng(3).standard_normal(10000).astype(np.float32)
    b = inputs.bf16_bits(x)
    w = inputs.bf16_bits_to_f32(b)
    assert np.all(inputs.bf16_bits(w) == b)
    # |x - round(x)| <= half an ulp of bf16 (2^-8 relative)
    assert np.all(np.abs(w - x) <= np.abs(x) * 2.0 ** -8 + 1e-45)


def test_problem_is_deterministic_and_seed_sensitive():
    a = inputs.make_problem(1, 2, 33, 32, inputs.BF16, causal=True, seed=5)
    b = inputs.make_problem(1, 2, 33, 32, inputs.BF16, causal=True, seed=5)
    c = inputs.make_problem(1, 2, 33, 32, inputs.BF16, causal=True, seed=6)
    assert a.sha256() == b.sha256() != c.sha256()
    assert a.q.shape == (2, 33, 32) and a.q.dtype == np.float32
    # bf16 problems hold exactly bf16-representable values
    for arr in (a.q, a.k, a.v):
        assert np.array_equal(inputs.bf16_bits_to_f32(inputs.bf16_bits(arr)), arr)


def test_q_scale_is_exact_power_of_two():
    base = inputs.make_problem(1, 1, 16, 32, inputs.BF16, seed=1)
    big = inputs.make_problem(1, 1, 16, 32, inputs.BF16, seed=1, q_scale=8.0)
    assert np.array_equal(big.q, base.q * 8)
    assert np.array_equal(big.k, base.k) and np.array_equal(big.v, base.v)
    with pytest.raises(ValueError):
        inputs.make_problem(1, 1, 4, 32, seed=0, q_scale=3.0)


def test_values_look_standard_normal():
    p = inputs.make_problem(1, 4, 256, 64, inputs.F32, seed=0)
    x = np.concatenate([p.q.ravel(), p.k.ravel(), p.v.ravel()])
    assert abs(x.mean()) < 0.01 and abs(x.std() - 1) < 0.01
