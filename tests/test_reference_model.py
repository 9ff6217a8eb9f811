"""CPU model of the bf16 flash kernel's reference tracking, run on the inputs
the GPU tests use to reach its correction and redo paths (flash_cases.py):
each case must reach the path its GPU test is meant to exercise.

The model follows the kernel's per-row rules (restated, not imported):
a wave owns 32 query rows; the first 64-key tile sets the reference to its
exact row maximum plus REF_MARGIN; every later tile up to the wave's last
(non-causal: all but the last tile, which takes an exact row maximum;
causal: through the wave's diagonal tile) computes probabilities
2^(x - m) against the current reference without a row maximum.  A lane holds
one row's 32 keys of a tile (keys 16c + 4h + {0..3, 8..11}, h the lane
half), and the wave's tile fails its check if any lane's sum exceeds
SPEC_LIMIT.  With every probability finite (below 2^128) it is corrected in
place: each row's reference moves up by the k with pmax 2^-k < 1.  An
infinite probability sends the whole query tile to the exact pass.  Scores
are taken in float64 from the same bf16-exact inputs (the kernel's fp32
rounding moves them by far less than the margins these cases leave).
"""
import re
from pathlib import Path

import numpy as np
import pytest

from tests.flash_cases import (REF_MARGIN, SPEC_LIMIT, diagonal_keys, first_tile_dominant, growing_keys,
                               sum_overflow_log2_score, sum_overflow_problem)

_HALF = (np.arange(64) // 4) % 2  # lane half holding each key of a tile


def _scores(p, bh, rows):
    """Scores of rows `rows` of slice bh in log2 units (scale log2(e)/sqrt(d)), causal mask applied."""
    x = (p.q[bh, rows].astype(np.float64) @ p.k[bh].astype(np.float64).T) * (np.log2(np.e) / np.sqrt(p.d))
    if p.causal:
        x = np.where(np.arange(p.S)[None, :] <= np.asarray(rows)[:, None], x, -np.inf)
    return x


def _wave(x, tiles):
    """Tracks one wave (rows of x) over steady tiles `tiles`; returns
    (tiles corrected in place, tiles with an infinite probability)."""
    m = np.max(x[:, :64], axis=1) + REF_MARGIN
    corrected, overflowed = [], []
    for t in tiles:
        xt = x[:, 64 * t:64 * t + 64]
        if xt.shape[1] < 64:
            xt = np.pad(xt, ((0, 0), (0, 64 - xt.shape[1])), constant_values=-np.inf)
        with np.errstate(over="ignore"):
            pt = np.exp2(xt - m[:, None])
        if np.any(pt >= 2.0 ** 128):
            overflowed.append(t)
            break  # the exact pass takes over
        lane = np.maximum(pt[:, _HALF == 0].sum(1), pt[:, _HALF == 1].sum(1))
        if np.any(lane > SPEC_LIMIT):
            corrected.append(t)
            m = m + np.maximum(np.floor(np.log2(np.max(pt, axis=1))) + 1, 0)
    return corrected, overflowed


def _track(p, heads=None):
    """(corrected tiles, overflowing waves, steady tiles) over every wave."""
    ntiles = (p.S + 63) // 64
    corr = over = steady = 0
    for bh in (range(p.BH) if heads is None else heads):
        for w0 in range(0, p.S, 32):
            rows = np.arange(w0, min(w0 + 32, p.S))
            x = _scores(p, bh, rows)
            last = min(ntiles, (w0 + 31) // 64 + 1) if p.causal else ntiles - 1
            c, o = _wave(x, range(1, last))
            corr, over, steady = corr + len(c), over + len(o), steady + max(last - 1, 0)
    return corr, over, steady


@pytest.mark.parametrize("d", [32, 64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_growing_keys_in_steps_are_corrected_in_place(d, causal):
    corr, over, steady = _track(growing_keys(d, causal, jump=False, S=1024))
    assert over == 0 and corr >= 0.05 * steady, (corr, over, steady)


@pytest.mark.parametrize("d", [32, 64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_growing_keys_at_once_overflow(d, causal):
    corr, over, steady = _track(growing_keys(d, causal, jump=True, S=1024))
    assert over > 0, (corr, over, steady)


def _diagonal_outcomes(p, heads):
    """Per wave at rows 448..511: did tile 7 (its diagonal tile, the item's
    last for these waves) get corrected in place, or overflow?"""
    got = []
    for bh in heads:
        for w0 in (448, 480):
            rows = np.arange(w0, w0 + 32)
            c, o = _wave(_scores(p, bh, rows), range(1, 8))
            got.append((7 in c, 7 in o))
    return got


@pytest.mark.parametrize("d", [32, 64, 128])
def test_diagonal_tile_x16_is_corrected_in_place_without_overflow(d):
    got = _diagonal_outcomes(diagonal_keys(d, 16.0), range(128))
    assert not any(o for _, o in got)
    assert sum(c for c, _ in got) >= 0.1 * len(got), sum(c for c, _ in got)


@pytest.mark.parametrize("d", [32, 64, 128])
def test_diagonal_tile_x256_overflows(d):
    got = _diagonal_outcomes(diagonal_keys(d, 256.0), range(16))
    assert all(o for _, o in got)


@pytest.mark.parametrize("d", [32, 64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_sum_overflow_case_has_finite_probabilities_and_an_infinite_sum(d, causal):
    x = sum_overflow_log2_score(d)
    # each later probability 2^x: finite in bf16 (largest finite 2^127 (2 - 2^-7)) and fp32
    assert 123.0 < x < 127.0 + np.log2(2.0 - 2.0 ** -7)
    assert 32 * 2.0 ** x >= 2.0 ** 128  # a lane's 32 of them overflow fp32
    p = sum_overflow_problem(d, causal)
    s = _scores(p, 0, np.arange(64, 128))  # rows whose tile 1 is a steady tile
    assert np.all(s[:, :64] == 0.0)  # tile 0 scores 0: the reference is REF_MARGIN
    vis = s[:, 64:128][np.isfinite(s[:, 64:128])]
    assert np.allclose(vis, x + REF_MARGIN)


@pytest.mark.parametrize("d", [32, 64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_first_tile_dominant_case_underflows_every_later_probability(d, causal):
    p = first_tile_dominant(d, causal)
    for bh in range(p.BH):
        rows = np.arange(64, p.S)  # rows with keys past the first tile
        x = _scores(p, bh, rows)
        m = np.max(x[:, :64], axis=1) + REF_MARGIN
        later = x[:, 64:] - m[:, None]
        assert np.all(later[np.isfinite(later)] < -126.0)  # below the fp32 normal range
        corr, over = _wave(x[:32], range(1, 4))
        assert corr == [] and over == []


def test_model_constants_match_the_kernel_source():
    """The model and the GPU cases restate the kernel's margin and sum limit:
    if either changes in the kernel, the cases above must be re-derived."""
    src = (Path(__file__).resolve().parents[1] / "transformer_attention_micro_amd" / "csrc" / "attn_flash.hip").read_text()
    margin = re.search(r"constexpr float kRefMargin = ([0-9.]+)f;", src)
    limit = re.search(r"constexpr float kSpecLimit = ([0-9.]+)f;", src)
    assert margin and limit
    assert float(margin.group(1)) == REF_MARGIN
    assert float(limit.group(1)) == SPEC_LIMIT
