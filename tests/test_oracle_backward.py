"""Pins of the oracle backward: central finite differences of the oracle forward,
the scalar brute-force chain rule, and gradient identities."""
import numpy as np
import pytest

import oracle
from oracle import MaskSpec, scalar

RNG = np.random.default_rng(11)

MASK_CASES = [
    ("none", {}), ("causal", {}), ("sliding_window", {"window": 2}),
    ("prefix_lm", {"prefix": 2}), ("block_diagonal", {}),
]


def _mask(kind, extra, nq, nk):
    if kind == "block_diagonal":
        dq = np.array([[0] * (nq // 2) + [1] * (nq - nq // 2)])
        dk = np.array([[0] * (nk // 2) + [1] * (nk - nk // 2)])
        return MaskSpec(kind, doc_q=dq, doc_k=dk)
    return MaskSpec(kind, **extra)


def _loss(q, k, v, do, **kw):
    o, _ = oracle.forward(q, k, v, **kw)
    return float(np.sum(np.nan_to_num(o) * do))


@pytest.mark.parametrize("kind,extra", MASK_CASES)
@pytest.mark.parametrize("softcap,slope", [(0.0, 0.0), (1.3, 0.0), (0.0, -0.2), (2.0, 0.1)])
@pytest.mark.parametrize("nq,nk", [(5, 5), (4, 6), (6, 3)])
def test_finite_differences(kind, extra, softcap, slope, nq, nk):
    d, dv = 3, 2
    q = RNG.standard_normal((1, nq, 1, d)); k = RNG.standard_normal((1, nk, 1, d))
    v = RNG.standard_normal((1, nk, 1, dv)); do = RNG.standard_normal((1, nq, 1, dv))
    kw = dict(scale=0.7, softcap=softcap, bias_slope=slope, mask=_mask(kind, extra, nq, nk))
    dq, dk, dvv, _, _ = oracle.backward(q, k, v, do, **kw)
    h = 1e-6
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dvv)):
        num = np.zeros_like(x)
        it = np.nditer(x, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            xp = x.copy(); xp[idx] += h
            xm = x.copy(); xm[idx] -= h
            args = {"q": q, "k": k, "v": v}
            args[name] = xp; lp = _loss(args["q"], args["k"], args["v"], do, **kw)
            args[name] = xm; lm = _loss(args["q"], args["k"], args["v"], do, **kw)
            num[idx] = (lp - lm) / (2 * h)
        scale = max(1.0, np.abs(num).max())
        assert np.abs(num - g).max() / scale < 1e-6, name


@pytest.mark.parametrize("kind,extra", MASK_CASES)
@pytest.mark.parametrize("softcap,slope", [(0.0, 0.0), (1.1, -0.25)])
def test_matches_scalar_chain_rule(kind, extra, softcap, slope):
    nq, nk, d, dv = 6, 7, 3, 4
    q = RNG.standard_normal((1, nq, 1, d)); k = RNG.standard_normal((1, nk, 1, d))
    v = RNG.standard_normal((1, nk, 1, dv)); do = RNG.standard_normal((1, nq, 1, dv))
    m = _mask(kind, extra, nq, nk)
    dq, dk, dvv, _, _ = oracle.backward(q, k, v, do, scale=0.9, softcap=softcap, bias_slope=slope, mask=m)
    mk = dict(extra)
    if kind == "block_diagonal":
        mk = {"doc_q": m.doc_q[0].tolist(), "doc_k": m.doc_k[0].tolist()}
    gq, gk, gv = scalar.attend_grad(q[0, :, 0].tolist(), k[0, :, 0].tolist(), v[0, :, 0].tolist(),
                                    do[0, :, 0].tolist(), 0.9, kind, softcap, slope, **mk)
    assert np.abs(dq[0, :, 0] - np.array(gq)).max() < 1e-12
    assert np.abs(dk[0, :, 0] - np.array(gk)).max() < 1e-12
    assert np.abs(dvv[0, :, 0] - np.array(gv)).max() < 1e-12


@pytest.mark.parametrize("kind,extra", MASK_CASES)
def test_key_gradients_sum_to_zero(kind, extra):
    # shifting every key by u adds a per-row constant to the scores: O is unchanged,
    # so sum_j dK_j = 0 (sum over each row of dS vanishes)
    nq, nk = 9, 9
    q = RNG.standard_normal((1, nq, 2, 4)); k = RNG.standard_normal((1, nk, 2, 4))
    v = RNG.standard_normal((1, nk, 2, 3)); do = RNG.standard_normal((1, nq, 2, 3))
    dq, dk, dv, _, _ = oracle.backward(q, k, v, do, bias_slope=-0.1, mask=_mask(kind, extra, nq, nk))
    assert np.abs(dk.sum(axis=1)).max() < 1e-12


def test_constant_v_gives_zero_dq_dk():
    q = RNG.standard_normal((1, 8, 1, 4)); k = RNG.standard_normal((1, 8, 1, 4))
    v = np.ones((1, 8, 1, 3)) * np.array([2.0, -1.0, 0.5]); do = RNG.standard_normal((1, 8, 1, 3))
    dq, dk, dv, _, _ = oracle.backward(q, k, v, do, mask=MaskSpec("causal"))
    assert np.abs(dq).max() < 1e-13 and np.abs(dk).max() < 1e-13


def test_dv_is_p_transpose_do():
    nq, nk = 5, 6
    q = RNG.standard_normal((1, nq, 1, 2)); k = RNG.standard_normal((1, nk, 1, 2))
    v = RNG.standard_normal((1, nk, 1, 3)); do = RNG.standard_normal((1, nq, 1, 3))
    _, _, dv, _, _ = oracle.backward(q, k, v, do, mask=MaskSpec("causal"))
    # P from the forward: O = P V for V = identity columns
    eye = np.eye(nk)[None, :, None, :]
    p, _ = oracle.forward(q, k, eye, mask=MaskSpec("causal"))
    assert np.abs(dv[0, :, 0] - p[0, :, 0].T @ do[0, :, 0]).max() < 1e-13


def test_fully_masked_rows_have_zero_gradient():
    q = RNG.standard_normal((1, 6, 1, 3)); k = RNG.standard_normal((1, 3, 1, 3))
    v = RNG.standard_normal((1, 3, 1, 2)); do = RNG.standard_normal((1, 6, 1, 2))
    dq, dk, dv, o, lse = oracle.backward(q, k, v, do, mask=MaskSpec("causal"))
    assert np.all(np.isfinite(dq)) and np.all(np.isfinite(dk)) and np.all(np.isfinite(dv))
    assert np.all(dq[0, :3] == 0.0) and np.all(lse[0, 0, :3] == -np.inf)
