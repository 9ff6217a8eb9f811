"""Pins for the fp64 oracle, independent of the oracle itself (CPU only).

Every pin comes from the definition on the kbench page ("The three GPU
kernels": O = softmax(Q K^T / sqrt(d)) V, [head, seq, dim] layout) or from
mathematics, never from the oracle's own output:
  * brute force in 50-digit decimal (a differently shaped evaluation) over
    exhaustive tiny grids and seeded tiny cases;
  * closed forms: two keys (sigmoid), S = 1, causal row 0, hand-worked
    rational cases in tests/golden/, the hardmax limit;
  * invariants: probability rows sum to one, identical value rows, Q = 0 gives
    the (prefix) mean, joint K/V row permutation without a mask, common key
    shift, causal row = unmasked attention over the prefix, head independence.
Shapes keep S != d and several heads so that a transposed operand or a wrong
head stride fails.
"""
import itertools
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
from tests._brute import brute_sdpa

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "closed_form_cases.json")


def rnd(shape, seed, scale=1.0):
    return (np.random.default_rng(seed).standard_normal(shape) * scale).astype(np.float32)


def grid(shape, seed, lo=-32, hi=32, denom=8.0):
    """Values on a coarse dyadic grid: sums and shifts of them stay exact in fp32."""
    return (np.random.default_rng(seed).integers(lo, hi + 1, size=shape) / denom).astype(np.float32)


# ---------------------------------------------------------------- brute force

@pytest.mark.parametrize("S,d", [(1, 1), (2, 1), (1, 2), (3, 1)])
@pytest.mark.parametrize("causal", [False, True])
def test_brute_force_exhaustive_ternary(S, d, causal):
    """All Q, K, V with entries in {-1, 0, 1} for tiny (S, d), batched as heads."""
    n = S * d
    combos = np.array(list(itertools.product((-1.0, 0.0, 1.0), repeat=3 * n)), dtype=np.float32)
    Q = combos[:, :n].reshape(-1, S, d)
    K = combos[:, n:2 * n].reshape(-1, S, d)
    V = combos[:, 2 * n:].reshape(-1, S, d)
    got = oracle.sdpa(Q, K, V, causal=causal)
    # brute force on a deterministic subset (the full grid for the smallest shapes)
    idx = range(len(combos)) if len(combos) <= 729 else np.random.default_rng(S * 10 + d).choice(len(combos), 729, replace=False)
    worst = 0.0
    for h in idx:
        ref = brute_sdpa(Q[h].tolist(), K[h].tolist(), V[h].tolist(), causal)
        worst = max(worst, float(np.max(np.abs(np.array(ref, dtype=np.float64) - got[h]))))
    assert worst <= 1e-13


@pytest.mark.parametrize("S,d", [(2, 2), (3, 2), (4, 3), (5, 4), (7, 3)])
@pytest.mark.parametrize("causal", [False, True])
def test_brute_force_seeded(S, d, causal):
    BH = 40
    Q, K, V = rnd((BH, S, d), 1), rnd((BH, S, d), 2), rnd((BH, S, d), 3, scale=2.0)
    got = oracle.sdpa(Q, K, V, causal=causal)
    for h in range(BH):
        ref = np.array(brute_sdpa(Q[h].tolist(), K[h].tolist(), V[h].tolist(), causal), dtype=np.float64)
        assert np.max(np.abs(ref - got[h])) <= 1e-13


def test_brute_force_explicit_scale():
    Q, K, V = rnd((3, 4, 3), 7), rnd((3, 4, 3), 8), rnd((3, 4, 3), 9)
    got = oracle.sdpa(Q, K, V, causal=False, scale=0.3)
    for h in range(3):
        ref = np.array(brute_sdpa(Q[h].tolist(), K[h].tolist(), V[h].tolist(), False, scale=0.3), dtype=np.float64)
        assert np.max(np.abs(ref - got[h])) <= 1e-13


# ---------------------------------------------------------------- closed forms

def test_two_keys_sigmoid_closed_form():
    """S = 2: O_i = V_0 + sigma(s_i1 - s_i0) (V_1 - V_0), s = q.k / sqrt(d)."""
    for seed in range(5):
        d = 4 + 2 * seed
        Q, K, V = rnd((2, 2, d), 10 + seed), rnd((2, 2, d), 20 + seed), rnd((2, 2, d), 30 + seed)
        got = oracle.sdpa(Q, K, V)
        q, k, v = Q.astype(np.float64), K.astype(np.float64), V.astype(np.float64)
        for h in range(2):
            for i in range(2):
                s0 = q[h, i] @ k[h, 0] / math.sqrt(d)
                s1 = q[h, i] @ k[h, 1] / math.sqrt(d)
                sig = 1.0 / (1.0 + math.exp(-(s1 - s0)))
                expect = v[h, 0] + sig * (v[h, 1] - v[h, 0])
                np.testing.assert_allclose(got[h, i], expect, rtol=0, atol=1e-14)


def test_single_key_and_causal_first_row():
    Q, K, V = rnd((3, 1, 5), 1), rnd((3, 1, 5), 2), rnd((3, 1, 5), 3)
    for causal in (False, True):
        np.testing.assert_array_equal(oracle.sdpa(Q, K, V, causal=causal), V.astype(np.float64))
    Q, K, V = rnd((3, 9, 5), 4), rnd((3, 9, 5), 5), rnd((3, 9, 5), 6)
    np.testing.assert_array_equal(oracle.sdpa(Q, K, V, causal=True)[:, 0], V[:, 0].astype(np.float64))


def _golden_value(x):
    if isinstance(x, str):
        if x.startswith("ln"):
            return float(np.float32(math.log(float(x[2:]))))
        return float(Fraction(x))
    return float(x)


def test_golden_closed_form_cases():
    spec = json.load(open(GOLDEN))
    for case in spec["cases"]:
        conv = lambda a: np.vectorize(_golden_value, otypes=[np.float64])(np.array(a, dtype=object))
        Q, K, V = (conv(case[n]).astype(np.float32) for n in ("q", "k", "v"))
        expect = conv(case["expected"])
        got = oracle.sdpa(Q, K, V, causal=case["causal"])
        np.testing.assert_allclose(got, expect, rtol=spec["tolerance"], atol=spec["tolerance"],
                                   err_msg=case["name"])


def test_hardmax_limit():
    """Q -> lambda Q with large lambda: a row whose largest scaled logit beats
    the runner-up by more than 40 puts weight < e^-40 on every other key, so
    it equals the value row of that key (hardmax)."""
    BH, S, d = 2, 12, 6
    K = rnd((BH, S, d), 11)
    V = rnd((BH, S, d), 12)
    Q = rnd((BH, S, d), 13) * np.float32(1e4)
    qd, kd = Q.astype(np.float64), K.astype(np.float64)
    for causal in (False, True):
        got = oracle.sdpa(Q, K, V, causal=causal)
        checked = 0
        for h in range(BH):
            for i in range(S):
                logits = kd[h] @ qd[h, i] / math.sqrt(d)
                if causal:
                    logits[i + 1:] = -np.inf
                if i == 0 and causal:
                    gap = np.inf
                else:
                    top2 = np.sort(logits)[::-1][:2]
                    gap = top2[0] - top2[1]
                if gap > 40:
                    np.testing.assert_allclose(got[h, i], V[h, int(np.argmax(logits))], rtol=0, atol=1e-12)
                    checked += 1
        assert checked >= 0.9 * BH * S


# ---------------------------------------------------------------- invariants

@pytest.mark.parametrize("causal", [False, True])
def test_probability_rows_sum_to_one_and_mask(causal):
    BH, S, d = 3, 37, 8
    Q, K, V = rnd((BH, S, d), 1, 2.0), rnd((BH, S, d), 2, 2.0), rnd((BH, S, d), 3)
    P = oracle.probs(Q, K, V, causal=causal)
    assert P.shape == (BH, S, S)
    assert np.all(P >= 0)
    np.testing.assert_allclose(P.sum(-1), 1.0, rtol=0, atol=1e-14)
    if causal:
        assert np.all(P[:, np.triu_indices(S, 1)[0], np.triu_indices(S, 1)[1]] == 0.0)
        assert np.all(P[:, np.tril_indices(S)[0], np.tril_indices(S)[1]] > 0.0)
    else:
        assert np.all(P > 0)
    # P.V reproduces O (O is the probability-weighted mean of the value rows)
    O = oracle.sdpa(Q, K, V, causal=causal)
    np.testing.assert_allclose(np.einsum("hij,hjd->hid", P, V.astype(np.float64)), O, atol=1e-13)


@pytest.mark.parametrize("causal", [False, True])
def test_identical_value_rows(causal):
    BH, S, d = 4, 29, 16
    Q, K = rnd((BH, S, d), 5, 3.0), rnd((BH, S, d), 6, 3.0)
    rows = rnd((BH, 1, d), 7)
    V = np.repeat(rows, S, axis=1)
    O = oracle.sdpa(Q, K, V, causal=causal)
    np.testing.assert_allclose(O, np.repeat(rows, S, axis=1).astype(np.float64), rtol=0, atol=1e-14)


@pytest.mark.parametrize("causal", [False, True])
def test_zero_query_gives_mean(causal):
    BH, S, d = 3, 21, 10
    Q = np.zeros((BH, S, d), np.float32)
    K, V = rnd((BH, S, d), 8), rnd((BH, S, d), 9)
    O = oracle.sdpa(Q, K, V, causal=causal)
    v = V.astype(np.float64)
    if causal:
        expect = np.cumsum(v, axis=1) / np.arange(1, S + 1)[None, :, None]
    else:
        expect = np.repeat(v.mean(axis=1, keepdims=True), S, axis=1)
    np.testing.assert_allclose(O, expect, rtol=0, atol=1e-14)


def test_joint_key_value_permutation():
    BH, S, d = 2, 33, 12
    Q, K, V = rnd((BH, S, d), 1), rnd((BH, S, d), 2), rnd((BH, S, d), 3)
    perm = np.random.default_rng(4).permutation(S)
    O = oracle.sdpa(Q, K, V)
    Op = oracle.sdpa(Q, K[:, perm], V[:, perm])
    np.testing.assert_allclose(Op, O, rtol=0, atol=1e-13)
    # negative control: under the causal mask the order of keys matters
    Oc = oracle.sdpa(Q, K, V, causal=True)
    Ocp = oracle.sdpa(Q, K[:, perm], V[:, perm], causal=True)
    assert np.max(np.abs(Ocp - Oc)) > 1e-2
    # and permuting K alone (not V) changes the unmasked result too
    assert np.max(np.abs(oracle.sdpa(Q, K[:, perm], V) - O)) > 1e-2


@pytest.mark.parametrize("causal", [False, True])
def test_common_key_shift(causal):
    """K_j -> K_j + c shifts every logit of a row by q.c/sqrt(d): O unchanged.
    Dyadic grid values keep the shifted keys exact; the large shift also
    exercises max subtraction (raw logits near 2e3 would overflow exp)."""
    BH, S, d = 2, 26, 8
    Q, K, V = grid((BH, S, d), 1), grid((BH, S, d), 2), grid((BH, S, d), 3)
    c = (np.random.default_rng(5).integers(-64, 65, size=(BH, 1, d))).astype(np.float32)
    O = oracle.sdpa(Q, K, V, causal=causal)
    Os = oracle.sdpa(Q, K + c, V, causal=causal)
    np.testing.assert_allclose(Os, O, rtol=0, atol=1e-11)


def test_causal_row_is_unmasked_attention_over_prefix():
    BH, S, d = 2, 19, 7
    Q, K, V = rnd((BH, S, d), 1), rnd((BH, S, d), 2), rnd((BH, S, d), 3)
    Oc = oracle.sdpa(Q, K, V, causal=True)
    for i in range(S):
        full = oracle.sdpa(np.repeat(Q[:, i:i + 1], i + 1, axis=1), K[:, :i + 1], V[:, :i + 1])
        np.testing.assert_allclose(Oc[:, i], full[:, 0], rtol=0, atol=1e-14)


def test_heads_are_independent_and_rows_api_matches():
    BH, S, d = 4, 17, 6
    Q, K, V = rnd((BH, S, d), 1), rnd((BH, S, d), 2), rnd((BH, S, d), 3)
    O = oracle.sdpa(Q, K, V, causal=True)
    K2, V2 = K.copy(), V.copy()
    K2[2] += 1.5
    V2[2] *= -3.0
    O2 = oracle.sdpa(Q, K2, V2, causal=True)
    np.testing.assert_array_equal(O2[[0, 1, 3]], O[[0, 1, 3]])
    assert np.max(np.abs(O2[2] - O[2])) > 1e-3
    rows = np.array([0, 5, S - 1, S, 2 * S + 3, BH * S - 1], dtype=np.int64)
    sub = oracle.sdpa(Q, K, V, causal=True, rows=rows)
    np.testing.assert_array_equal(sub, O.reshape(BH * S, d)[rows])
    Psub = oracle.probs(Q, K, V, causal=True, rows=rows)
    np.testing.assert_array_equal(Psub, oracle.probs(Q, K, V, causal=True).reshape(BH * S, S)[rows])


def test_thread_count_does_not_change_result():
    Q, K, V = rnd((3, 40, 16), 1), rnd((3, 40, 16), 2), rnd((3, 40, 16), 3)
    a = oracle.sdpa(Q, K, V, causal=True, nthreads=1)
    b = oracle.sdpa(Q, K, V, causal=True, nthreads=7)
    np.testing.assert_array_equal(a, b)


def test_rejects_bad_arguments():
    Q = rnd((1, 4, 2), 1)
    with pytest.raises(ValueError):
        oracle.sdpa(Q, Q[:, :3], Q)
    with pytest.raises(ValueError):
        oracle.sdpa(Q, Q, Q, rows=[4])
