"""GPU parity of the split-KV forward (partials + LSE-weighted combine)."""
import numpy as np
import pytest

import oracle
from block_sparse_attention_fmha_amd import synth
from tests.gpu_util import announce, check_bf16, host, mask_pair, to_dev

pytestmark = pytest.mark.gpu


def run_split(q, k, v, splits, gmask=None):
    import torch
    import block_sparse_attention_fmha_amd as fa
    out, lse = fa.fmha_fwd_splitkv(q, k, v, splits, mask=gmask)
    torch.cuda.synchronize()
    return out, lse


@pytest.mark.parametrize("splits", [1, 2, 4, 8, 16, 64])
@pytest.mark.parametrize("nq,nk,d,kind", [(1, 1000, 128, "none"), (3, 777, 64, "causal"),
                                          (1, 4096, 128, "sliding_window")])
def test_splitkv_small(splits, nq, nk, d, kind):
    seed = synth.case_seed(9, 500 + nk + d)
    q, k, v = synth.attention_inputs(seed, 2, nq, nk, 3, d, d, "bf16")
    om, gm = mask_pair(kind, 2, nq, nk, window=700)
    announce(f"splitkv seed={seed} Nq={nq} Nk={nk} D={d} mask={kind} splits={splits}")
    out, lse = run_split(to_dev(q), to_dev(k), to_dev(v), splits, gm)
    o_ref, l_ref = oracle.forward(q.values, k.values, v.values, mask=om)
    check_bf16("O", host(out), o_ref)
    check_bf16("LSE", host(lse), l_ref)


@pytest.fixture(scope="module")
def decode_inputs():
    # B=8 H=32 Nq=1 Nk=32768 D=128, no mask: generated once for every split count
    seed = synth.case_seed(5, 0)
    q, k, v = synth.attention_inputs(seed, 8, 1, 32768, 32, 128, 128, "bf16")
    tq, tk, tv = to_dev(q), to_dev(k), to_dev(v)
    pairs = [(0, 0), (3, 17), (7, 31)]
    refs = {bh: oracle.forward_bh(q.values[bh[0], :, bh[1]], k.values[bh[0], :, bh[1]],
                                  v.values[bh[0], :, bh[1]], np.arange(1), bh[0], bh[1], 1, 32768,
                                  scale=1 / np.sqrt(128.0)) for bh in pairs}
    return seed, (tq, tk, tv), refs


@pytest.mark.parametrize("splits", [1, 2, 4, 8, 16])
def test_splitkv_full_size(decode_inputs, splits):
    seed, (tq, tk, tv), refs = decode_inputs
    announce(f"splitkv full size seed={seed} B=8 H=32 Nk=32768 splits={splits}")
    out, lse = run_split(tq, tk, tv, splits)
    o, l = host(out), host(lse)
    for (b, h), (o_ref, l_ref) in refs.items():
        check_bf16(f"O[{b},{h}]", o[b, :, h], o_ref)
        check_bf16(f"LSE[{b},{h}]", l[b, h], l_ref)


def _gqa_inputs(seed, B, nq, nk, H, Hkv, d):
    # Q with H heads, K / V with Hkv heads, from the shared seeded generator
    q = synth.attention_inputs(seed, B, nq, nk, H, d, d, "bf16")[0]
    _, k, v = synth.attention_inputs(seed + 1, B, nq, nk, Hkv, d, d, "bf16")
    return q, k, v


@pytest.mark.parametrize("splits", [1, 3, 16])
@pytest.mark.parametrize("H,Hkv", [(8, 2), (8, 4), (6, 2), (8, 1), (12, 1)])
@pytest.mark.parametrize("nq,nk,d,kind", [(1, 1000, 128, "none"), (3, 777, 64, "causal")])
def test_splitkv_grouped_heads_small(splits, H, Hkv, nq, nk, d, kind):
    # grouped-query (Hkv divides H) and multi-query (Hkv = 1) heads: query head h reads
    # K/V head h // (H / Hkv)
    seed = synth.case_seed(9, 700 + 10 * H + Hkv + d)
    q, k, v = _gqa_inputs(seed, 2, nq, nk, H, Hkv, d)
    om, gm = mask_pair(kind, 2, nq, nk)
    announce(f"splitkv grouped heads seed={seed} H={H} Hkv={Hkv} Nq={nq} Nk={nk} D={d} mask={kind} splits={splits}")
    out, lse = run_split(to_dev(q), to_dev(k), to_dev(v), splits, gm)
    o_ref, l_ref = oracle.forward(q.values, k.values, v.values, mask=om)
    check_bf16("O", host(out), o_ref)
    check_bf16("LSE", host(lse), l_ref)


@pytest.mark.parametrize("Hkv,splits", [(8, 1), (8, 16), (1, 16)])
def test_splitkv_grouped_heads_full_size(Hkv, splits):
    # B=8 H=32 Nq=1 Nk=32768 D=128 with 8 (groups of 4) or 1 (multi-query) K/V heads
    seed = synth.case_seed(5, 10 + Hkv)
    q, k, v = _gqa_inputs(seed, 8, 1, 32768, 32, Hkv, 128)
    announce(f"splitkv grouped heads full size seed={seed} B=8 H=32 Hkv={Hkv} Nk=32768 splits={splits}")
    out, lse = run_split(to_dev(q), to_dev(k), to_dev(v), splits)
    o, l = host(out), host(lse)
    for b, h in ((0, 0), (2, 5), (5, 18), (7, 31)):
        g = oracle.kv_head(h, 32, Hkv)
        o_ref, l_ref = oracle.forward_bh(q.values[b, :, h], k.values[b, :, g], v.values[b, :, g], np.arange(1),
                                         b, h, 1, 32768, scale=1 / np.sqrt(128.0))
        check_bf16(f"O[{b},{h}]", o[b, :, h], o_ref)
        check_bf16(f"LSE[{b},{h}]", l[b, h], l_ref)


@pytest.mark.parametrize("Hkv", [8, 2, 1])
def test_splitkv_no_keys(Hkv):
    # an empty K / V cache: every split is empty, so O = 0 and LSE = -inf (the combine of
    # empty partials); output buffers start as NaN
    import torch
    import block_sparse_attention_fmha_amd as fa
    dev = torch.device("cuda:0")
    q = synth.attention_inputs(synth.case_seed(9, 990 + Hkv), 2, 1, 1, 8, 128, 128, "bf16")[0]
    none = torch.empty(2, 0, Hkv, 128, device=dev, dtype=torch.bfloat16)
    out = torch.full((2, 1, 8, 128), float("nan"), device=dev, dtype=torch.bfloat16)
    lse = torch.full((2, 8, 1), float("nan"), device=dev, dtype=torch.float32)
    announce(f"splitkv Nk=0 B=2 H=8 Hkv={Hkv} splits=8")
    out, lse = fa.fmha_fwd_splitkv(to_dev(q), none, none, 8, out=out, lse=lse)
    torch.cuda.synchronize()
    assert torch.all(out == 0) and torch.all(torch.isneginf(lse))


@pytest.mark.parametrize("H,Hkv,nq,kind,splits", [(16, 2, 1, "none", 4), (16, 1, 2, "sliding_window", 3),
                                                  (8, 2, 1, "causal", 2), (8, 2, 3, "none", 1)])
def test_splitkv_grouped_heads_d64(H, Hkv, nq, kind, splits):
    # head dim 64 with groups of 4 (>= 1024 keys per split), 8 and 16 query heads per K/V
    # head: the matrix-core decode path at D = 64, against the oracle element-wise
    seed = synth.case_seed(9, 900 + 10 * H + Hkv + nq)
    q, k, v = _gqa_inputs(seed, 2, nq, 5000, H, Hkv, 64)
    om, gm = mask_pair(kind, 2, nq, 5000, window=700)
    announce(f"splitkv grouped heads D=64 seed={seed} H={H} Hkv={Hkv} Nq={nq} Nk=5000 mask={kind} splits={splits}")
    out, lse = run_split(to_dev(q), to_dev(k), to_dev(v), splits, gm)
    o_ref, l_ref = oracle.forward(q.values, k.values, v.values, mask=om)
    check_bf16("O", host(out), o_ref)
    check_bf16("LSE", host(lse), l_ref)
