"""fmha_fwd_splitkv_noalloc (library-owned scratch, no allocation in the call) against
fmha_fwd_splitkv (caller workspace) through the C ABI: two calls in a row, the second with a
smaller input, each bitwise equal to the workspace entry point on the same inputs (same
kernels), and within the bf16 tolerance of the oracle."""
import numpy as np
import pytest

import oracle
from block_sparse_attention_fmha_amd import synth
from tests.gpu_util import announce, check_bf16, host, to_dev

pytestmark = pytest.mark.gpu


def _case(seed, B, H, Hkv, Nk, splits):
    import torch
    import block_sparse_attention_fmha_amd as fa
    q = synth.attention_inputs(seed, B, 1, Nk, H, 128, 128, "bf16")[0]
    _, k, v = synth.attention_inputs(seed + 1, B, 1, Nk, Hkv, 128, 128, "bf16")
    tq, tk, tv = to_dev(q), to_dev(k), to_dev(v)
    announce(f"splitkv noalloc B={B} H={H} Hkv={Hkv} Nk={Nk} splits={splits}")
    o1, l1 = fa.fmha_fwd_splitkv_noalloc(tq, tk, tv, splits)
    o2, l2 = fa.fmha_fwd_splitkv(tq, tk, tv, splits)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    ro, rl = oracle.forward(q.values, k.values, v.values)
    check_bf16("O", host(o1), ro)
    check_bf16("LSE", host(l1), rl)


def test_noalloc_two_calls_second_smaller():
    import block_sparse_attention_fmha_amd as fa
    assert fa.load_library().fmha_fwd_splitkv_noalloc_max_bytes() == 16 << 20
    _case(synth.case_seed(5, 900), 4, 16, 4, 9000, 16)    # grouped heads, the larger call
    _case(synth.case_seed(5, 901), 1, 8, 8, 1000, 4)      # then a smaller one, multi-head
