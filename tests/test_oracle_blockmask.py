"""Pins of the block-mask tile classification and index lists: closed-form tile
counts, pure-Python element enumeration, and list/transposed-list consistency."""
import numpy as np
import pytest

import oracle
from oracle import MaskSpec
from oracle.blockmask import EMPTY, FULL, PARTIAL, classify_tiles


def test_causal_counts_closed_form():
    # 8192 / 128 -> 64 x 64 tiles: the diagonal is partial, strictly below is full
    cls = classify_tiles(MaskSpec("causal"), 1, 1, 8192, 8192, 128, 128)[0, 0]
    assert (cls == PARTIAL).sum() == 64
    assert (cls == FULL).sum() == 64 * 63 // 2
    assert (cls == EMPTY).sum() == 64 * 63 // 2
    r, c = np.indices(cls.shape)
    assert np.all(cls[r == c] == PARTIAL) and np.all(cls[r > c] == FULL)


def _window_closed_form(n, t, w):
    nt = n // t
    out = np.zeros((nt, nt), np.int8)
    for r in range(nt):
        for c in range(nt):
            qlo, qhi, klo, khi = r * t, r * t + t - 1, c * t, c * t + t - 1
            if klo > qhi or khi < qlo - w:
                out[r, c] = EMPTY
            elif khi <= qlo and klo >= qhi - w:
                out[r, c] = FULL
            else:
                out[r, c] = PARTIAL
    return out


@pytest.mark.parametrize("n,t,w", [(8192, 128, 2730), (1024, 64, 100), (512, 128, 128)])
def test_window_classes_closed_form(n, t, w):
    cls = classify_tiles(MaskSpec("sliding_window", window=w), 1, 1, n, n, t, t)[0, 0]
    assert np.array_equal(cls, _window_closed_form(n, t, w))


def test_prefix_classes_closed_form():
    n, t, p = 8192, 128, 1024
    cls = classify_tiles(MaskSpec("prefix_lm", prefix=p), 1, 1, n, n, t, t)[0, 0]
    r, c = np.indices(cls.shape)
    want = np.where(c < p // t, FULL, np.where(r > c, FULL, np.where(r == c, PARTIAL, EMPTY)))
    assert np.array_equal(cls, want)


def _brute(kind, nq, nk, tm, tn, **mk):
    from oracle.scalar import _visible
    nqt, nkt = -(-nq // tm), -(-nk // tn)
    out = np.zeros((nqt, nkt), np.int8)
    for r in range(nqt):
        for c in range(nkt):
            vis = tot = 0
            for i in range(r * tm, min(nq, r * tm + tm)):
                for j in range(c * tn, min(nk, c * tn + tn)):
                    tot += 1
                    vis += _visible(kind, i, j, nq, nk, **mk)
            out[r, c] = EMPTY if vis == 0 else (FULL if vis == tot else PARTIAL)
    return out


@pytest.mark.parametrize("nq,nk,tm,tn", [(37, 53, 8, 16), (64, 40, 16, 8), (50, 50, 7, 9)])
@pytest.mark.parametrize("kind,extra", [("none", {}), ("causal", {}), ("sliding_window", {"window": 11}),
                                        ("prefix_lm", {"prefix": 13}), ("block_diagonal", {})])
def test_classes_match_element_enumeration(nq, nk, tm, tn, kind, extra):
    if kind == "block_diagonal":
        rng = np.random.default_rng(nq * nk)
        dq = np.sort(rng.integers(0, 4, nq)); dk = np.sort(rng.integers(0, 4, nk))
        ms = MaskSpec(kind, doc_q=dq[None], doc_k=dk[None])
        extra = {"doc_q": dq.tolist(), "doc_k": dk.tolist()}
    else:
        ms = MaskSpec(kind, **extra)
    cls = classify_tiles(ms, 1, 1, nq, nk, tm, tn)[0, 0]
    assert np.array_equal(cls, _brute(kind, nq, nk, tm, tn, **extra))


def test_lists_layout_and_transpose_consistency():
    ms = MaskSpec("sliding_window", window=20)
    L = oracle.build_lists(ms, 2, 1, 100, 90, 16, 8)
    nqt, nkt = 7, 12
    assert L.partial_idx.shape == (2, 1, nqt, nkt) and L.t_partial_idx.shape == (2, 1, nkt, nqt)
    for cnt, idx in ((L.partial_cnt, L.partial_idx), (L.full_cnt, L.full_idx),
                     (L.t_partial_cnt, L.t_partial_idx), (L.t_full_cnt, L.t_full_idx)):
        for b in range(2):
            for r in range(idx.shape[2]):
                n = cnt[b, 0, r]
                assert np.all(np.diff(idx[b, 0, r, :n]) > 0)
                assert np.all(idx[b, 0, r, n:] == -1)
    cls = classify_tiles(ms, 2, 1, 100, 90, 16, 8)
    for b in range(2):
        pairs = {(r, c) for r in range(nqt) for c in L.partial_idx[b, 0, r, : L.partial_cnt[b, 0, r]]}
        tpairs = {(r, c) for c in range(nkt) for r in L.t_partial_idx[b, 0, c, : L.t_partial_cnt[b, 0, c]]}
        assert pairs == tpairs == set(zip(*np.nonzero(cls[b, 0] == PARTIAL)))
        assert (L.partial_cnt[b, 0].sum() + L.full_cnt[b, 0].sum()
                + (cls[b, 0] == EMPTY).sum()) == nqt * nkt
