"""Pins of the split-KV partials and the LSE-weighted combine."""
import math

import numpy as np
import pytest

import oracle
from oracle import MaskSpec
from oracle.attention import split_ranges

RNG = np.random.default_rng(3)


@pytest.mark.parametrize("splits", [1, 2, 4, 8, 16])
@pytest.mark.parametrize("tile_n", [1, 4, 16])
@pytest.mark.parametrize("nq", [1, 3])
def test_combine_equals_unsplit(splits, tile_n, nq):
    nk = 37
    q = RNG.standard_normal((2, nq, 2, 4)); k = RNG.standard_normal((2, nk, 2, 4))
    v = RNG.standard_normal((2, nk, 2, 3))
    o, lse = oracle.combine_partials(oracle.split_partials(q, k, v, splits, tile_n))
    o_ref, lse_ref = oracle.forward(q, k, v)
    assert np.abs(o - o_ref).max() < 1e-13 and np.abs(lse - lse_ref).max() < 1e-13


def test_combine_with_causal_empty_rows():
    q = RNG.standard_normal((1, 5, 1, 4)); k = RNG.standard_normal((1, 3, 1, 4))
    v = RNG.standard_normal((1, 3, 1, 2))
    o, lse = oracle.combine_partials(oracle.split_partials(q, k, v, 4, 1, mask=MaskSpec("causal")))
    o_ref, lse_ref = oracle.forward(q, k, v, mask=MaskSpec("causal"))
    assert np.array_equal(o[0, :2], np.zeros((2, 1, 2)))
    assert np.all(lse[0, 0, :2] == -np.inf)
    f = np.isfinite(lse_ref)
    assert np.abs(o - o_ref).max() < 1e-13 and np.abs(lse[f] - lse_ref[f]).max() < 1e-13


def test_two_chunk_merge_closed_form():
    # chunk 1: one key with score a, value x; chunk 2: one key with score b, value y
    a, b, x, y = 0.3, -1.2, 2.0, -5.0
    parts = [(np.full((1, 1, 1, 1), x), np.full((1, 1, 1), a)),
             (np.full((1, 1, 1, 1), y), np.full((1, 1, 1), b))]
    o, lse = oracle.combine_partials(parts)
    w = math.exp(a) / (math.exp(a) + math.exp(b))
    assert o.item() == pytest.approx(w * x + (1 - w) * y, abs=1e-15)
    assert lse.item() == pytest.approx(math.log(math.exp(a) + math.exp(b)), abs=1e-15)


def test_all_empty_partials():
    parts = [(np.zeros((1, 1, 1, 2)), np.full((1, 1, 1), -np.inf))] * 3
    o, lse = oracle.combine_partials(parts)
    assert np.all(o == 0.0) and np.all(lse == -np.inf)


def test_split_ranges_partition():
    for nk in (1, 37, 128, 32768):
        for s in (1, 2, 4, 8, 16):
            for t in (1, 64, 128):
                r = split_ranges(nk, s, t)
                assert r[0][0] == 0 and r[-1][1] == nk
                assert all(r[i][1] == r[i + 1][0] for i in range(s - 1))
                assert all(lo % t == 0 or lo == nk for lo, _ in r)
