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
