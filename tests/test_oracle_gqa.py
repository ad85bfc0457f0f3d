"""Pins of the oracle's grouped-query attention (query heads sharing K/V heads), each
against a formulation that does not use the head mapping under test."""
import numpy as np
import pytest

import oracle


def _rand(rng, *shape):
    return rng.standard_normal(shape)


@pytest.mark.parametrize("H,Hkv", [(4, 2), (6, 3), (8, 1), (4, 4)])
@pytest.mark.parametrize("kind", ["none", "causal"])
def test_gqa_equals_mha_on_repeated_kv(H, Hkv, kind):
    # sharing a K/V head is the same as giving every query head its own copy of it
    rng = np.random.default_rng(H * 10 + Hkv)
    B, Nq, Nk, D = 2, 5, 7, 4
    q, k, v = _rand(rng, B, Nq, H, D), _rand(rng, B, Nk, Hkv, D), _rand(rng, B, Nk, Hkv, D)
    m = oracle.MaskSpec(kind)
    o, lse = oracle.forward(q, k, v, mask=m)
    G = H // Hkv
    o_r, lse_r = oracle.forward(q, np.repeat(k, G, axis=2), np.repeat(v, G, axis=2), mask=m)
    assert np.allclose(o, o_r, rtol=0, atol=1e-13) and np.allclose(lse, lse_r, rtol=0, atol=1e-13)


def test_mqa_every_head_reads_the_one_kv_head():
    rng = np.random.default_rng(7)
    B, Nq, Nk, H, D = 1, 4, 6, 3, 5
    q, k, v = _rand(rng, B, Nq, H, D), _rand(rng, B, Nk, 1, D), _rand(rng, B, Nk, 1, D)
    o, lse = oracle.forward(q, k, v)
    for h in range(H):
        ob, lb = oracle.forward(q[:, :, h:h + 1], k, v)
        assert np.allclose(o[:, :, h], ob[:, :, 0], atol=1e-14) and np.allclose(lse[:, h], lb[:, 0], atol=1e-14)


def test_kv_head_mapping_and_rejection():
    assert [oracle.kv_head(h, 8, 2) for h in range(8)] == [0, 0, 0, 0, 1, 1, 1, 1]
    assert [oracle.kv_head(h, 6, 6) for h in range(6)] == list(range(6))
    with pytest.raises(ValueError):
        oracle.kv_head(0, 6, 4)
    rng = np.random.default_rng(1)
    with pytest.raises(ValueError):
        oracle.forward(_rand(rng, 1, 2, 6, 4), _rand(rng, 1, 3, 4, 4), _rand(rng, 1, 3, 4, 4))


def test_gqa_split_partials_combine_to_the_forward():
    rng = np.random.default_rng(11)
    B, Nq, Nk, H, Hkv, D = 2, 1, 200, 8, 2, 8
    q, k, v = _rand(rng, B, Nq, H, D), _rand(rng, B, Nk, Hkv, D), _rand(rng, B, Nk, Hkv, D)
    o_ref, lse_ref = oracle.forward(q, k, v)
    for splits in (1, 3, 5):
        o, lse = oracle.combine_partials(oracle.split_partials(q, k, v, splits, 64))
        assert np.allclose(o, o_ref, atol=1e-12) and np.allclose(lse, lse_ref, atol=1e-12)


@pytest.mark.parametrize("kind", ["none", "causal"])
def test_gqa_backward_matches_finite_differences(kind):
    # central differences of the grouped-head forward (fp64) for dQ, dK and dV
    rng = np.random.default_rng(21)
    B, Nq, Nk, H, Hkv, D = 1, 3, 4, 4, 2, 2
    q, k, v, do = (rng.standard_normal(s) for s in ((B, Nq, H, D), (B, Nk, Hkv, D), (B, Nk, Hkv, D), (B, Nq, H, D)))
    m = oracle.MaskSpec(kind)
    dq, dk, dv, _, _ = oracle.backward(q, k, v, do, mask=m, bias_slope=0.1)

    def loss(q_, k_, v_):
        o, _ = oracle.forward(q_, k_, v_, mask=m, bias_slope=0.1)
        return float((o * do).sum())

    eps = 1e-6
    for arr, grad, which in ((q, dq, 0), (k, dk, 1), (v, dv, 2)):
        num = np.zeros_like(arr)
        for idx in np.ndindex(arr.shape):
            args_p = [q.copy(), k.copy(), v.copy()]
            args_m = [q.copy(), k.copy(), v.copy()]
            args_p[which][idx] += eps
            args_m[which][idx] -= eps
            num[idx] = (loss(*args_p) - loss(*args_m)) / (2 * eps)
        assert np.abs(num - grad).max() <= 1e-6 * max(1.0, np.abs(num).max())
