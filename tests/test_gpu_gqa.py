"""GPU parity of the forward with grouped K/V heads (query head h reads K/V head
h // (H / Hkv)) against the fp64 oracle: bf16 (masks, softcap, bias, MLA-shaped heads,
block-sparse lists), fp32 (D 64 and the 1024 wide head) and packed variable-length
sequences."""
import numpy as np
import pytest

import oracle
from block_sparse_attention_fmha_amd import synth
from tests.gpu_util import announce, check_bf16, check_fp32, host, mask_pair, to_dev

pytestmark = pytest.mark.gpu


def _inputs(seed, B, nq, nk, H, Hkv, dqk, dv, dtype):
    q = synth.attention_inputs(seed, B, nq, nk, H, dqk, dv, dtype)[0]
    _, k, v = synth.attention_inputs(seed + 1, B, nq, nk, Hkv, dqk, dv, dtype)
    return q, k, v


CASES = [
    # (dtype, B, Nq, Nk, H, Hkv, Dqk, Dv, mask, softcap, slope, lists)
    ("bf16", 2, 300, 500, 8, 2, 128, 128, "causal", 0.0, 0.0, None),
    ("bf16", 1, 257, 257, 6, 3, 64, 64, "none", 30.0, 0.0, None),
    ("bf16", 1, 384, 384, 4, 1, 192, 128, "prefix_lm", 0.0, -0.01, None),
    ("bf16", 2, 512, 512, 4, 2, 128, 128, "sliding_window", 0.0, -0.01, (128, 128)),
    ("fp32", 1, 150, 170, 6, 3, 64, 64, "causal", 0.0, 0.0, None),
    ("fp32", 1, 100, 130, 4, 2, 1024, 1024, "none", 0.0, 0.0, None),
]


@pytest.mark.parametrize("case", range(len(CASES)))
def test_fwd_grouped_heads(case):
    import torch
    import block_sparse_attention_fmha_amd as fa
    dtype, B, nq, nk, H, Hkv, dqk, dv, kind, cap, slope, lists = CASES[case]
    seed = synth.case_seed(9, 950 + case)
    q, k, v = _inputs(seed, B, nq, nk, H, Hkv, dqk, dv, dtype)
    om, gm = mask_pair(kind, B, nq, nk, window=100, prefix=50)
    announce(f"fwd grouped heads seed={seed} {dtype} B={B} Nq={nq} Nk={nk} H={H} Hkv={Hkv} D={dqk}/{dv} "
             f"mask={kind} softcap={cap} bias={slope} lists={lists}")
    bs = fa.build_block_mask(gm, B, nq, nk, *lists) if lists else None
    out, lse = fa.fmha_fwd(to_dev(q), to_dev(k), to_dev(v), mask=gm, softcap=cap, bias_slope=slope, block_sparse=bs)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.forward(q.values, k.values, v.values, mask=om, softcap=cap, bias_slope=slope)
    chk = check_fp32 if dtype == "fp32" else check_bf16
    chk("O", host(out), o_ref)
    chk("LSE", host(lse), l_ref)


def test_varlen_grouped_heads():
    import torch
    import block_sparse_attention_fmha_amd as fa
    lq, lk, H, Hkv, D = [300, 1, 700, 129], [300, 40, 700, 200], 4, 2, 128
    cu_q = np.concatenate([[0], np.cumsum(lq)]).astype(np.int32)
    cu_k = np.concatenate([[0], np.cumsum(lk)]).astype(np.int32)
    seed = synth.case_seed(9, 990)
    q, k, v = _inputs(seed, 1, int(cu_q[-1]), int(cu_k[-1]), H, Hkv, D, D, "bf16")
    dev = torch.device("cuda:0")
    announce(f"varlen fwd grouped heads seed={seed} H={H} Hkv={Hkv}")
    out, lse = fa.fmha_fwd_varlen(q.to_torch(dev)[0], k.to_torch(dev)[0], v.to_torch(dev)[0],
                                  torch.from_numpy(cu_q).to(dev), torch.from_numpy(cu_k).to(dev), max(lq), max(lk),
                                  mask=fa.Mask("causal"))
    torch.cuda.synchronize()
    # per sequence through the (grouped-head) oracle forward
    o_ref = np.zeros((int(cu_q[-1]), H, D))
    l_ref = np.full((H, int(cu_q[-1])), -np.inf)
    for b in range(len(lq)):
        qs, qe, ks, ke = cu_q[b], cu_q[b + 1], cu_k[b], cu_k[b + 1]
        ob, lb = oracle.forward(q.values[:, qs:qe], k.values[:, ks:ke], v.values[:, ks:ke],
                                mask=oracle.MaskSpec("causal"))
        o_ref[qs:qe], l_ref[:, qs:qe] = ob[0], lb[0]
    check_bf16("O", host(out), o_ref)
    check_bf16("LSE", host(lse), l_ref)


BWD_CASES = [
    # (B, Nq, Nk, H, Hkv, Dqk, Dv, mask, softcap, slope, lists)
    (2, 300, 500, 8, 2, 128, 128, "causal", 0.0, 0.0, None),
    (1, 384, 384, 6, 3, 64, 64, "sliding_window", 30.0, 0.0, None),
    (1, 256, 384, 4, 1, 192, 128, "prefix_lm", 0.0, -0.01, None),
    (2, 512, 512, 4, 2, 128, 128, "causal", 0.0, -0.01, (128, 128)),
]


@pytest.mark.parametrize("case", range(len(BWD_CASES)))
def test_bwd_grouped_heads(case):
    import torch
    import block_sparse_attention_fmha_amd as fa
    from tests.gpu_util import check_grad
    B, nq, nk, H, Hkv, dqk, dv, kind, cap, slope, lists = BWD_CASES[case]
    seed = synth.case_seed(9, 960 + case)
    q, k, v = _inputs(seed, B, nq, nk, H, Hkv, dqk, dv, "bf16")
    do = synth.attention_inputs(seed + 2, B, nq, nk, H, dqk, dv, "bf16", with_dout=True)[3]
    om, gm = mask_pair(kind, B, nq, nk, window=100, prefix=50)
    announce(f"bwd grouped heads seed={seed} B={B} Nq={nq} Nk={nk} H={H} Hkv={Hkv} D={dqk}/{dv} mask={kind} "
             f"softcap={cap} bias={slope} lists={lists}")
    bs = fa.build_block_mask(gm, B, nq, nk, *lists) if lists else None
    tq, tk, tv, tdo = to_dev(q), to_dev(k), to_dev(v), to_dev(do)
    out, lse = fa.fmha_fwd(tq, tk, tv, mask=gm, softcap=cap, bias_slope=slope, block_sparse=bs)
    dq, dk, dv_ = fa.fmha_bwd(tq, tk, tv, out, lse, tdo, mask=gm, softcap=cap, bias_slope=slope, block_sparse=bs)
    torch.cuda.synchronize()
    ref = oracle.backward(q.values, k.values, v.values, do.values, mask=om, softcap=cap, bias_slope=slope)
    for name, got, want in (("dQ", dq, ref[0]), ("dK", dk, ref[1]), ("dV", dv_, ref[2])):
        check_grad(name, host(got), want)
    # deterministic: a second run is bitwise identical
    dq2, dk2, dv2 = fa.fmha_bwd(tq, tk, tv, out, lse, tdo, mask=gm, softcap=cap, bias_slope=slope, block_sparse=bs)
    torch.cuda.synchronize()
    assert torch.equal(dq, dq2) and torch.equal(dk, dk2) and torch.equal(dv_, dv2)
