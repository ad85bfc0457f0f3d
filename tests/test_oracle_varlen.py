"""Pins of the oracle's packed variable-length forward, each against the batched forward
on the same rows (a formulation without offsets)."""
import numpy as np
import pytest

import oracle


@pytest.mark.parametrize("kind", ["none", "causal", "sliding_window", "prefix_lm"])
def test_equal_lengths_equal_the_batched_forward(kind):
    rng = np.random.default_rng(3)
    B, Nq, Nk, H, D = 3, 5, 7, 2, 4
    q, k, v = rng.standard_normal((B, Nq, H, D)), rng.standard_normal((B, Nk, H, D)), rng.standard_normal((B, Nk, H, D))
    m = oracle.MaskSpec(kind, window=2, prefix=3)
    o_ref, l_ref = oracle.forward(q, k, v, mask=m, bias_slope=-0.1)
    cu_q, cu_k = np.arange(B + 1) * Nq, np.arange(B + 1) * Nk
    o, lse = oracle.forward_varlen(q.reshape(B * Nq, H, D), k.reshape(B * Nk, H, D), v.reshape(B * Nk, H, D),
                                   cu_q, cu_k, mask=m, bias_slope=-0.1)
    assert np.array_equal(o, o_ref.reshape(B * Nq, H, D))
    assert np.array_equal(lse, l_ref.transpose(1, 0, 2).reshape(H, B * Nq))


def test_each_sequence_is_its_own_problem():
    rng = np.random.default_rng(5)
    H, D = 2, 8
    lq, lk = [4, 1, 6, 0, 3], [9, 2, 6, 3, 0]
    cu_q, cu_k = np.concatenate([[0], np.cumsum(lq)]), np.concatenate([[0], np.cumsum(lk)])
    q, k, v = (rng.standard_normal((n, H, D)) for n in (cu_q[-1], cu_k[-1], cu_k[-1]))
    m = oracle.MaskSpec("causal")
    o, lse = oracle.forward_varlen(q, k, v, cu_q, cu_k, mask=m)
    for b in range(len(lq)):
        qs, qe, ks, ke = cu_q[b], cu_q[b + 1], cu_k[b], cu_k[b + 1]
        if qe == qs:
            continue
        if ke == ks:   # no keys at all: O = 0, LSE = -inf
            assert np.all(o[qs:qe] == 0) and np.all(np.isneginf(lse[:, qs:qe]))
            continue
        ob, lb = oracle.forward(q[None, qs:qe], k[None, ks:ke], v[None, ks:ke], mask=m)
        assert np.array_equal(o[qs:qe], ob[0]) and np.array_equal(lse[:, qs:qe], lb[0])


@pytest.mark.parametrize("kind", ["causal", "sliding_window"])
def test_backward_equal_lengths_equal_the_batched_backward(kind):
    rng = np.random.default_rng(9)
    B, Nq, Nk, H, D = 2, 6, 5, 2, 3
    q, k, v, do = (rng.standard_normal(s) for s in ((B, Nq, H, D), (B, Nk, H, D), (B, Nk, H, D), (B, Nq, H, D)))
    m = oracle.MaskSpec(kind, window=2)
    ref = oracle.backward(q, k, v, do, mask=m, bias_slope=0.05)
    cu_q, cu_k = np.arange(B + 1) * Nq, np.arange(B + 1) * Nk
    got = oracle.backward_varlen(q.reshape(-1, H, D), k.reshape(-1, H, D), v.reshape(-1, H, D),
                                 do.reshape(-1, H, D), cu_q, cu_k, mask=m, bias_slope=0.05)
    for g, r in zip(got[:4], ref[:4]):
        assert np.array_equal(g, r.reshape(g.shape))
    assert np.array_equal(got[4], ref[4].transpose(1, 0, 2).reshape(H, B * Nq))


def _packed(rng, lq, lk, H=2, D=4):
    cu_q, cu_k = np.concatenate([[0], np.cumsum(lq)]), np.concatenate([[0], np.cumsum(lk)])
    q, k, v, do = (rng.standard_normal((n, H, D)) for n in (cu_q[-1], cu_k[-1], cu_k[-1], cu_q[-1]))
    return cu_q, cu_k, q, k, v, do


@pytest.mark.parametrize("kind", ["causal", "sliding_window", "prefix_lm"])
def test_seqused_equal_to_the_span_changes_nothing(kind):
    rng = np.random.default_rng(21)
    lq, lk = [5, 0, 3, 7], [6, 2, 0, 7]
    cu_q, cu_k, q, k, v, do = _packed(rng, lq, lk)
    m = oracle.MaskSpec(kind, window=2, prefix=2)
    a = oracle.forward_varlen(q, k, v, cu_q, cu_k, mask=m, bias_slope=0.1)
    b = oracle.forward_varlen(q, k, v, cu_q, cu_k, mask=m, bias_slope=0.1, seqused_q=np.array(lq),
                              seqused_k=np.array(lk))
    assert all(np.array_equal(x, y) for x, y in zip(a, b))
    a = oracle.backward_varlen(q, k, v, do, cu_q, cu_k, mask=m, softcap=1.5)
    b = oracle.backward_varlen(q, k, v, do, cu_q, cu_k, mask=m, softcap=1.5, seqused_q=np.array(lq),
                               seqused_k=np.array(lk))
    assert all(np.array_equal(x, y) for x, y in zip(a, b))


@pytest.mark.parametrize("kind", ["none", "causal", "sliding_window"])
def test_seqused_shorter_than_the_span_equals_the_truncated_sequences(kind):
    # used prefixes of each span vs. a packing that holds only those prefixes: the used rows
    # must agree exactly and every row past a used length is left out (NaN)
    rng = np.random.default_rng(22)
    lq, lk = [6, 4, 5, 3], [7, 5, 4, 3]
    uq, uk = [4, 0, 5, 2], [7, 3, 0, 1]
    cu_q, cu_k, q, k, v, do = _packed(rng, lq, lk)
    m = oracle.MaskSpec(kind, window=1)
    rows_q = np.concatenate([np.arange(cu_q[b], cu_q[b] + uq[b]) for b in range(4)]).astype(int)
    rows_k = np.concatenate([np.arange(cu_k[b], cu_k[b] + uk[b]) for b in range(4)]).astype(int)
    tcu_q, tcu_k = np.concatenate([[0], np.cumsum(uq)]), np.concatenate([[0], np.cumsum(uk)])
    o, lse = oracle.forward_varlen(q, k, v, cu_q, cu_k, mask=m, seqused_q=np.array(uq), seqused_k=np.array(uk))
    to, tl = oracle.forward_varlen(q[rows_q], k[rows_k], v[rows_k], tcu_q, tcu_k, mask=m)
    assert np.array_equal(o[rows_q], to) and np.array_equal(lse[:, rows_q], tl)
    rest_q = np.setdiff1d(np.arange(cu_q[-1]), rows_q)
    assert np.all(np.isnan(o[rest_q])) and np.all(np.isnan(lse[:, rest_q]))
    g = oracle.backward_varlen(q, k, v, do, cu_q, cu_k, mask=m, seqused_q=np.array(uq), seqused_k=np.array(uk))
    t = oracle.backward_varlen(q[rows_q], k[rows_k], v[rows_k], do[rows_q], tcu_q, tcu_k, mask=m)
    assert np.array_equal(g[0][rows_q], t[0])
    assert np.array_equal(g[1][rows_k], t[1]) and np.array_equal(g[2][rows_k], t[2])
    rest_k = np.setdiff1d(np.arange(cu_k[-1]), rows_k)
    assert np.all(np.isnan(g[0][rest_q])) and np.all(np.isnan(g[1][rest_k])) and np.all(np.isnan(g[2][rest_k]))


def test_seqused_outside_the_span_is_rejected():
    rng = np.random.default_rng(23)
    cu_q, cu_k, q, k, v, _ = _packed(rng, [3, 2], [3, 2])
    with pytest.raises(ValueError):
        oracle.forward_varlen(q, k, v, cu_q, cu_k, seqused_q=np.array([4, 2]))
    with pytest.raises(ValueError):
        oracle.forward_varlen(q, k, v, cu_q, cu_k, seqused_k=np.array([1, -1]))
