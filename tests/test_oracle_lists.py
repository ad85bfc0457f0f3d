"""Pins of the oracle's block-sparse list semantics: per-head lists and set membership.

Source: "Enable 2CTA for SM100 block-sparse backward", section "Summary" (a listed FULL
tile is attended without the element mask, a PARTIAL tile applies it, an unlisted tile is
skipped) and the fuzz tester's block_sparse_tensors ("Testing Testing Testing"), which
carry a head axis. The readings pinned here (list layout reading in the design notes):
  * lists with one mask head serve every head; with H mask heads, head h reads its own;
  * a list row is a set: an entry given twice counts once, a tile in both lists of a row
    is full, an index outside [0, nKt) names no tile, a count is clamped to [0, nKt].

Closed forms: with Q = 0 every visible score is 0, so LSE_i = ln(number of visible keys
of row i) and O_i is the mean of the visible V rows. With V row j = e_{tile(j)} (one-hot
of j's key tile), O_i is the share of row i's visible keys that each key tile supplies.
The expected counts below are worked out by hand from the window predicate
i - W <= j <= i (W = 1, Nq = Nk = 8, 4 x 4 tiles) and the listed tiles.
"""
from __future__ import annotations

import math

import numpy as np
import pytest

import oracle
from oracle import MaskSpec

N, T = 8, 4             # 8 queries / keys, 4 x 4 sparse tiles: 2 x 2 tiles
WINDOW = MaskSpec("sliding_window", window=1)


def _lists(pc, pi, fc, fi):
    a = lambda x: np.asarray(x, np.int32)
    return oracle.BlockLists(T, T, a(pc), a(pi), a(fc), a(fi), None, None, None, None)


def _hand_lists():
    """B = 1, two mask heads.
    head 0: partial count -1 over entries [0, 1] (a negative count lists nothing, it does
            not mean "all but the last"), full count 0: every tile skipped.
    head 1: query tile 0: partial [0, 0] (a repeated entry), full count 5 over [1, 1]
            (count clamped to the row length; repeated entry);
            query tile 1: partial [1, 0], full [0, -1] (tile 0 in both lists: full;
            -1 names no tile, it is not "the last tile")."""
    pc = [[[-1, -1], [2, 2]]]
    pi = [[[[0, 1], [0, 1]], [[0, 0], [1, 0]]]]
    fc = [[[0, 0], [5, 2]]]
    fi = [[[[-1, -1], [-1, -1]], [[1, 1], [0, -1]]]]
    return _lists(pc, pi, fc, fi)


# visible keys of each row of head 1, by key tile (tile 0, tile 1), counted by hand:
#   rows 0-3: tile 0 partial under the window (row 0: {0}; rows 1-3: {i-1, i}), tile 1 full
#   rows 4-7: tile 0 full (in both lists), tile 1 partial (row 4: {4}; rows 5-7: {i-1, i})
HEAD1_COUNTS = [(1, 4), (2, 4), (2, 4), (2, 4), (4, 1), (4, 2), (4, 2), (4, 2)]


def _onehot_inputs(H=2):
    q = np.zeros((1, N, H, 2))
    k = np.random.default_rng(5).standard_normal((1, N, H, 2))   # irrelevant: Q = 0
    v = np.zeros((1, N, H, 2))
    for j in range(N):
        v[0, j, :, j // T] = 1.0
    return q, k, v


def test_per_head_lists_and_set_semantics_closed_form():
    q, k, v = _onehot_inputs()
    o, lse = oracle.forward(q, k, v, mask=WINDOW, lists=_hand_lists())
    # head 0: nothing listed -> every row empty: O = 0, LSE = -inf
    assert np.all(o[0, :, 0] == 0.0)
    assert np.all(np.isneginf(lse[0, 0]))
    # head 1: LSE = ln(count), O = per-tile share of the visible keys
    for i, (c0, c1) in enumerate(HEAD1_COUNTS):
        n = c0 + c1
        assert abs(lse[0, 1, i] - math.log(n)) < 1e-14, (i, lse[0, 1, i], n)
        assert abs(o[0, i, 1, 0] - c0 / n) < 1e-14 and abs(o[0, i, 1, 1] - c1 / n) < 1e-14, i


def test_single_head_lists_broadcast_over_heads():
    # the head-1 lists alone (one mask head) give every head head 1's answer
    L = _hand_lists()
    one = _lists(L.partial_cnt[:, 1:], L.partial_idx[:, 1:], L.full_cnt[:, 1:], L.full_idx[:, 1:])
    q, k, v = _onehot_inputs(H=3)
    o, lse = oracle.forward(q, k, v, mask=WINDOW, lists=one)
    for h in range(3):
        for i, (c0, c1) in enumerate(HEAD1_COUNTS):
            assert abs(lse[0, h, i] - math.log(c0 + c1)) < 1e-14
            assert abs(o[0, i, h, 1] - c1 / (c0 + c1)) < 1e-14


def _empty_and_full(first_full: bool):
    """Two mask heads: one lists every tile as full, the other lists nothing."""
    pc = np.zeros((1, 2, 2), np.int32); pi = np.full((1, 2, 2, 2), -1, np.int32)
    fc = np.zeros((1, 2, 2), np.int32); fi = np.full((1, 2, 2, 2), -1, np.int32)
    hf = 0 if first_full else 1
    fc[0, hf] = 2
    fi[0, hf] = [[0, 1], [1, 0]]   # any order
    return _lists(pc, pi, fc, fi)


@pytest.mark.parametrize("first_full", [True, False])
def test_per_head_full_equals_dense_and_empty_is_zero_forward_and_backward(first_full):
    rng = np.random.default_rng(11)
    q, k, v, do = (rng.standard_normal((1, N, 2, 3)) for _ in range(4))
    L = _empty_and_full(first_full)
    hf, he = (0, 1) if first_full else (1, 0)
    # the element mask must not matter on full tiles: use one that hides most keys
    causal = MaskSpec("causal")
    o, lse = oracle.forward(q, k, v, mask=causal, lists=L)
    o_d, lse_d = oracle.forward(q, k, v)             # dense, no mask
    assert np.abs(o[0, :, hf] - o_d[0, :, hf]).max() < 1e-14
    assert np.abs(lse[0, hf] - lse_d[0, hf]).max() < 1e-14
    assert np.all(o[0, :, he] == 0.0) and np.all(np.isneginf(lse[0, he]))
    dq, dk, dv, _, _ = oracle.backward(q, k, v, do, mask=causal, lists=L)
    gq, gk, gv, _, _ = oracle.backward(q, k, v, do)
    for got, ref in ((dq, gq), (dk, gk), (dv, gv)):
        assert np.abs(got[0, :, hf] - ref[0, :, hf]).max() < 1e-13
        assert np.all(got[0, :, he] == 0.0)


def test_out_of_range_entries_add_nothing():
    # a row listing only out-of-range entries (and a count past the row length over them)
    # is an empty row
    L = _lists([[[2, 0]]], [[[[-1, 7], [-1, -1]]]], [[[9, 0]]], [[[[2, -2], [-1, -1]]]])
    q, k, v = _onehot_inputs(H=1)
    o, lse = oracle.forward(q, k, v, lists=L)
    assert np.all(np.isneginf(lse[0, 0])) and np.all(o == 0.0)
