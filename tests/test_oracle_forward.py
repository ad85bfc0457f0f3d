"""Pins of the oracle forward against closed forms, invariants and the scalar brute force.

Each pin is chosen so that a plausible slip (scale 1/D instead of 1/sqrt(D), a
transposed product, log base 2, top-left instead of bottom-right causal alignment,
an off-by-one window end, a dropped bias or softcap) fails at least one of them.
"""
import math

import numpy as np
import pytest

import oracle
from oracle import MaskSpec, scalar
from oracle.attention import streaming_forward_bh
from oracle.masks import fuzz_window

RNG = np.random.default_rng(7)


def _one(q, k, v, **kw):
    """Forward on [Nq,D], [Nk,D], [Nk,Dv] arrays (B=H=1)."""
    o, l = oracle.forward(np.asarray(q)[None, :, None], np.asarray(k)[None, :, None],
                          np.asarray(v)[None, :, None], **kw)
    return o[0, :, 0], l[0, 0]


# ---------------------------------------------------------------- closed forms

def test_two_key_closed_form():
    # D=4 -> scale 1/2. s0 = 0.5*2 = 1, s1 = 0.5*(1*-1 + 0) = -0.5
    q = [[1.0, 0.0, 0.0, 0.0]]
    k = [[2.0, 0.0, 0.0, 0.0], [-1.0, 3.0, 0.0, 0.0]]
    v = [[1.0, 2.0], [3.0, -4.0]]
    o, lse = _one(q, k, v)
    e0, e1 = math.exp(1.0), math.exp(-0.5)
    p0 = e0 / (e0 + e1)
    assert o[0] == pytest.approx([p0 * 1 + (1 - p0) * 3, p0 * 2 + (1 - p0) * -4], abs=1e-15)
    assert lse[0] == pytest.approx(math.log(e0 + e1), abs=1e-15)


def test_explicit_scale_is_used():
    q = [[1.0, 1.0]]
    k = [[1.0, 0.0], [0.0, 0.0]]
    v = [[1.0], [0.0]]
    o, lse = _one(q, k, v, scale=3.0)      # s = [3, 0]
    assert o[0, 0] == pytest.approx(math.exp(3) / (math.exp(3) + 1), abs=1e-15)
    assert lse[0] == pytest.approx(math.log(math.exp(3) + 1), abs=1e-15)


def test_softcap_closed_form():
    q = [[2.0, 0.0, 0.0, 0.0]]
    k = [[3.0, 0.0, 0.0, 0.0], [0.0, 0.0, 0.0, 0.0]]    # s_pre = [3, 0]
    v = [[1.0], [0.0]]
    c = 2.0
    o, lse = _one(q, k, v, softcap=c)
    s0 = c * math.tanh(3.0 / c)
    assert o[0, 0] == pytest.approx(math.exp(s0) / (math.exp(s0) + 1.0), abs=1e-15)
    assert lse[0] == pytest.approx(math.log(math.exp(s0) + 1.0), abs=1e-15)


def test_relative_bias_closed_form():
    # all raw scores zero: S = sigma*|i-j|
    q = np.zeros((3, 2)); k = np.zeros((3, 2)); v = np.eye(3)
    sig = -0.7
    o, lse = _one(q, k, v, bias_slope=sig)
    for i in range(3):
        w = np.array([math.exp(sig * abs(i - j)) for j in range(3)])
        assert o[i] == pytest.approx(w / w.sum(), abs=1e-15)
        assert lse[i] == pytest.approx(math.log(w.sum()), abs=1e-15)


def test_causal_bottom_right_alignment_and_empty_rows():
    q = RNG.standard_normal((4, 3)); k = RNG.standard_normal((2, 3)); v = RNG.standard_normal((2, 5))
    o, lse = _one(q, k, v, mask=MaskSpec("causal"))
    # delta = Nk - Nq = -2: rows 0, 1 see nothing; row 2 sees key 0; row 3 sees keys 0, 1
    assert np.all(o[:2] == 0.0) and np.all(lse[:2] == -np.inf)
    assert o[2] == pytest.approx(v[0], abs=1e-15)
    s = k @ q[2] / math.sqrt(3)
    assert lse[2] == pytest.approx(s[0], abs=1e-14)
    # a single decode query sees every key
    o1, _ = _one(q[:1], np.vstack([k, k]), np.vstack([v, v]), mask=MaskSpec("causal"))
    o2, _ = _one(q[:1], np.vstack([k, k]), np.vstack([v, v]))
    assert o1 == pytest.approx(o2, abs=1e-15)


def test_causal_row0_is_v0_and_lse_is_s00():
    q = RNG.standard_normal((6, 4)); k = RNG.standard_normal((6, 4)); v = RNG.standard_normal((6, 3))
    o, lse = _one(q, k, v, mask=MaskSpec("causal"))
    assert o[0] == pytest.approx(v[0], abs=1e-15)
    assert lse[0] == pytest.approx(q[0] @ k[0] / 2.0, abs=1e-14)


def test_window_bounds_inclusive():
    n = 6
    q = np.zeros((n, 2)); k = np.zeros((n, 2)); v = np.eye(n)
    o, _ = _one(q, k, v, mask=MaskSpec("sliding_window", window=1))
    for i in range(n):
        want = np.zeros(n)
        lo = max(0, i - 1)
        want[lo:i + 1] = 1.0 / (i + 1 - lo)
        assert o[i] == pytest.approx(want, abs=1e-15)


def test_prefix_lm_and_block_diagonal_patterns():
    n = 5
    q = np.zeros((n, 2)); k = np.zeros((n, 2)); v = np.eye(n)
    o, _ = _one(q, k, v, mask=MaskSpec("prefix_lm", prefix=2))
    for i in range(n):
        vis = [j for j in range(n) if j < 2 or j <= i]
        assert o[i] == pytest.approx(np.isin(np.arange(n), vis) / len(vis), abs=1e-15)
    docs = np.array([[0, 0, 1, 1, 1]])
    o, _ = _one(q, k, v, mask=MaskSpec("block_diagonal", doc_q=docs, doc_k=docs))
    for i in range(n):
        vis = docs[0] == docs[0, i]
        assert o[i] == pytest.approx(vis / vis.sum(), abs=1e-15)


def test_fuzz_window_rule():
    assert fuzz_window(8192, 8192) == 2730
    assert fuzz_window(100, 1000) == 64


# ---------------------------------------------------------------- invariants

def _rand(nq, nk, d, dv):
    return (RNG.standard_normal((2, nq, 3, d)), RNG.standard_normal((2, nk, 3, d)),
            RNG.standard_normal((2, nk, 3, dv)))


MASKS = [MaskSpec("none"), MaskSpec("causal"), MaskSpec("sliding_window", window=5),
         MaskSpec("prefix_lm", prefix=4)]


@pytest.mark.parametrize("mask", MASKS, ids=lambda m: m.kind)
def test_weights_sum_to_one_and_constant_v(mask):
    q, k, v = _rand(17, 17, 8, 4)
    v[:] = np.array([1.5, -2.0, 0.25, 7.0])
    o, _ = oracle.forward(q, k, v, mask=mask)
    assert np.abs(o - v[:, :1]).max() < 1e-14


@pytest.mark.parametrize("mask", MASKS, ids=lambda m: m.kind)
def test_convex_hull_and_linearity(mask):
    q, k, v = _rand(13, 13, 8, 4)
    o, _ = oracle.forward(q, k, v, mask=mask)
    assert np.all(o <= v.max(axis=1, keepdims=True) + 1e-12)
    assert np.all(o >= v.min(axis=1, keepdims=True) - 1e-12)
    v2 = RNG.standard_normal(v.shape)
    o2, _ = oracle.forward(q, k, v2, mask=mask)
    o3, _ = oracle.forward(q, k, 2.0 * v - 3.0 * v2, mask=mask)
    assert np.abs(o3 - (2.0 * o - 3.0 * o2)).max() < 1e-12


def test_key_shift_changes_lse_not_o():
    q, k, v = _rand(9, 9, 4, 3)
    u = RNG.standard_normal(4)
    o, lse = oracle.forward(q, k, v, mask=MaskSpec("causal"))
    o2, lse2 = oracle.forward(q, k + u, v, mask=MaskSpec("causal"))
    assert np.abs(o - o2).max() < 1e-12
    shift = np.einsum("bqhd,d->bhq", q, u) / 2.0
    assert np.abs(lse2 - lse - shift).max() < 1e-12


def test_key_permutation_invariance():
    q, k, v = _rand(7, 11, 4, 3)
    perm = RNG.permutation(11)
    o, lse = oracle.forward(q, k, v)
    o2, lse2 = oracle.forward(q, k[:, perm], v[:, perm])
    assert np.abs(o - o2).max() < 1e-13 and np.abs(lse - lse2).max() < 1e-13


def test_single_key_gives_v0():
    q, k, v = _rand(5, 1, 4, 3)
    o, lse = oracle.forward(q, k, v)
    assert np.abs(o - v[:, :1]).max() < 1e-15


def test_mask_reductions():
    q, k, v = _rand(12, 12, 4, 3)
    causal = oracle.forward(q, k, v, mask=MaskSpec("causal"))
    none = oracle.forward(q, k, v)
    for a, b in [(oracle.forward(q, k, v, mask=MaskSpec("sliding_window", window=12)), causal),
                 (oracle.forward(q, k, v, mask=MaskSpec("prefix_lm", prefix=0)), causal),
                 (oracle.forward(q, k, v, mask=MaskSpec("prefix_lm", prefix=12)), none)]:
        assert np.abs(a[0] - b[0]).max() < 1e-14 and np.abs(a[1] - b[1]).max() < 1e-14
    one_doc = np.zeros((2, 12), np.int32)
    bd = oracle.forward(q, k, v, mask=MaskSpec("block_diagonal", doc_q=one_doc, doc_k=one_doc))
    assert np.abs(bd[0] - none[0]).max() < 1e-14
    unit = np.tile(np.arange(12, dtype=np.int32), (2, 1))
    bd1 = oracle.forward(q, k, v, mask=MaskSpec("block_diagonal", doc_q=unit, doc_k=unit))
    assert np.abs(bd1[0] - v).max() < 1e-15


def test_softcap_limit_is_off():
    q, k, v = _rand(6, 6, 4, 3)
    a = oracle.forward(q, k, v, softcap=1e9)
    b = oracle.forward(q, k, v)
    assert np.abs(a[0] - b[0]).max() < 1e-12


def test_all_full_block_lists_equal_dense_and_mask_lists_equal_mask():
    q, k, v = _rand(40, 40, 4, 3)
    none = MaskSpec("none")
    lists = oracle.build_lists(none, 2, 1, 40, 40, 16, 8)
    assert np.all(lists.partial_cnt == 0)
    a = oracle.forward(q, k, v, lists=lists, mask=MaskSpec("causal"))  # element mask unused on full tiles
    b = oracle.forward(q, k, v)
    assert np.abs(a[0] - b[0]).max() < 1e-15
    for m in MASKS:
        lists = oracle.build_lists(m, 2, 1, 40, 40, 16, 8)
        a = oracle.forward(q, k, v, lists=lists, mask=m)
        b = oracle.forward(q, k, v, mask=m)
        assert np.abs(a[0] - b[0]).max() < 1e-15


# ---------------------------------------------------------------- cross-formulations

CASES = [
    (5, 5, 4, 3, "none", {}), (6, 4, 3, 2, "causal", {}), (3, 8, 4, 4, "causal", {}),
    (7, 7, 2, 3, "sliding_window", {"window": 2}), (5, 9, 3, 3, "sliding_window", {"window": 3}),
    (8, 8, 4, 2, "prefix_lm", {"prefix": 3}), (6, 6, 4, 4, "block_diagonal", {}),
]


@pytest.mark.parametrize("nq,nk,d,dv,kind,extra", CASES)
@pytest.mark.parametrize("softcap,slope", [(0.0, 0.0), (1.5, 0.0), (0.0, -0.3)])
def test_vectorised_matches_scalar(nq, nk, d, dv, kind, extra, softcap, slope):
    q = RNG.standard_normal((1, nq, 1, d)); k = RNG.standard_normal((1, nk, 1, d))
    v = RNG.standard_normal((1, nk, 1, dv))
    docs = None
    if kind == "block_diagonal":
        docs = np.array([[0, 0, 1, 1, 1, 2]])
        extra = {"doc_q": docs[0].tolist(), "doc_k": docs[0].tolist()}
    scale = 0.8
    ms = MaskSpec(kind, window=extra.get("window", 0), prefix=extra.get("prefix", 0),
                  doc_q=docs, doc_k=docs)
    o, lse = oracle.forward(q, k, v, scale=scale, softcap=softcap, bias_slope=slope, mask=ms)
    so, sl = scalar.attend(q[0, :, 0].tolist(), k[0, :, 0].tolist(), v[0, :, 0].tolist(), scale,
                           kind, softcap, slope, **extra)
    so, sl = np.array(so), np.array(sl)
    assert np.abs(o[0, :, 0] - so).max() < 1e-12
    fin = np.isfinite(sl)
    assert np.array_equal(np.isfinite(lse[0, 0]), fin)
    assert np.abs(lse[0, 0][fin] - sl[fin]).max(initial=0) < 1e-12


@pytest.mark.parametrize("tile", [1, 3, 8, 64])
@pytest.mark.parametrize("mask", MASKS + [MaskSpec("causal")], ids=lambda m: m.kind)
def test_streaming_merge_matches_materialised(tile, mask):
    nq, nk = 11, 19
    q = RNG.standard_normal((nq, 4)); k = RNG.standard_normal((nk, 4)); v = RNG.standard_normal((nk, 3))
    a = oracle.forward_bh(q, k, v, np.arange(nq), 0, 0, nq, nk, scale=0.5, softcap=2.0, mask=mask)
    b = streaming_forward_bh(q, k, v, np.arange(nq), 0, 0, nq, nk, tile, scale=0.5, softcap=2.0, mask=mask)
    assert np.abs(a[0] - b[0]).max() < 1e-12
    assert np.array_equal(np.isfinite(a[1]), np.isfinite(b[1]))
    f = np.isfinite(a[1])
    assert np.abs(a[1][f] - b[1][f]).max(initial=0) < 1e-12


def test_row_subset_matches_full():
    q, k, v = _rand(30, 30, 4, 3)
    rows = [0, 7, 29]
    a = oracle.forward(q, k, v, mask=MaskSpec("causal"), rows=rows, heads=[1])
    b = oracle.forward(q, k, v, mask=MaskSpec("causal"))
    assert np.abs(a[0][:, rows, 1] - b[0][:, rows, 1]).max() < 1e-14
    assert np.abs(a[1][:, 1, rows] - b[1][:, 1, rows]).max() < 1e-14
