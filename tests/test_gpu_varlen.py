"""GPU parity of the packed variable-length forward (fmha_fwd_varlen) against the fp64
oracle's per-sequence definition."""
import numpy as np
import pytest

import oracle
from block_sparse_attention_fmha_amd import synth
from tests.gpu_util import announce, check_bf16, check_grad, host

pytestmark = pytest.mark.gpu


def _run(seed, lq, lk, H, dqk, dv, kind, window=0, prefix=0, softcap=0.0, slope=0.0, backward=False):
    import torch
    import block_sparse_attention_fmha_amd as fa
    cu_q = np.concatenate([[0], np.cumsum(lq)]).astype(np.int32)
    cu_k = np.concatenate([[0], np.cumsum(lk)]).astype(np.int32)
    # packed rows from the shared seeded generator: [1, total, H, D] -> [total, H, D]
    q = synth.attention_inputs(seed, 1, int(cu_q[-1]), int(cu_k[-1]), H, dqk, dv, "bf16", with_dout=True)
    qv, kv, vv, dov = (x.values[0] for x in q)
    dev = torch.device("cuda:0")
    tq, tk, tv, tdo = (x.to_torch(dev)[0] for x in q)
    announce(f"varlen fwd seed={seed} seqs={len(lq)} total_q={cu_q[-1]} total_k={cu_k[-1]} H={H} "
             f"D={dqk}/{dv} mask={kind} W={window} P={prefix} softcap={softcap} bias={slope}")
    out, lse = fa.fmha_fwd_varlen(tq, tk, tv, torch.from_numpy(cu_q).to(dev), torch.from_numpy(cu_k).to(dev),
                                  max(lq), max(lk), mask=fa.Mask(kind, window=window, prefix=prefix),
                                  softcap=softcap, bias_slope=slope)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.forward_varlen(qv, kv, vv, cu_q, cu_k, softcap=softcap, bias_slope=slope,
                                         mask=oracle.MaskSpec(kind, window=window, prefix=prefix))
    check_bf16("O", host(out), o_ref)
    check_bf16("LSE", host(lse), l_ref)
    if backward:
        tcu_q, tcu_k = torch.from_numpy(cu_q).to(dev), torch.from_numpy(cu_k).to(dev)
        dq, dk, dv_ = fa.fmha_bwd_varlen(tq, tk, tv, out, lse, tdo, tcu_q, tcu_k, max(lq), max(lk),
                                         mask=fa.Mask(kind, window=window, prefix=prefix), softcap=softcap,
                                         bias_slope=slope)
        torch.cuda.synchronize()
        ref = oracle.backward_varlen(qv, kv, vv, dov, cu_q, cu_k, softcap=softcap, bias_slope=slope,
                                     mask=oracle.MaskSpec(kind, window=window, prefix=prefix))
        for name, got, want in (("dQ", dq, ref[0]), ("dK", dk, ref[1]), ("dV", dv_, ref[2])):
            check_grad(name, host(got), want)


CASES = [
    # (query lengths, key lengths, H, Dqk, Dv, mask, window, prefix, softcap, slope)
    ([300, 1, 700, 256, 129], [300, 1, 700, 256, 129], 2, 128, 128, "causal", 0, 0, 0.0, 0.0),
    ([513, 40, 1000], [769, 200, 1000], 2, 128, 128, "causal", 0, 0, 0.0, 0.0),        # Nk > Nq per sequence
    ([257, 600], [129, 100], 2, 128, 128, "causal", 0, 0, 0.0, 0.0),                  # rows with no key
    ([640, 333, 77], [640, 333, 77], 2, 64, 64, "sliding_window", 100, 0, 30.0, 0.0),
    ([384, 500, 2], [384, 500, 2], 2, 128, 128, "prefix_lm", 0, 100, 0.0, -0.01),
    ([255, 385], [385, 255], 2, 192, 128, "none", 0, 0, 0.0, -0.05),
    ([1000, 0, 300], [1000, 50, 0], 1, 128, 128, "none", 0, 0, 0.0, 0.0),             # empty sequences
]


@pytest.mark.parametrize("case", range(len(CASES)))
def test_varlen_forward(case):
    lq, lk, H, dqk, dv, kind, w, p, cap, slope = CASES[case]
    _run(synth.case_seed(9, 800 + case), lq, lk, H, dqk, dv, kind, w, p, cap, slope)


def test_varlen_documents_of_the_block_sparse_workload():
    # the block-diagonal workload's documents (B=2 rows of N=8192, lengths 256..2048) packed
    # as one sequence each, no mask inside a document
    docs = synth.document_ids(synth.case_seed(3, 2), 2, 8192)
    lens = [int(c) for b in range(2) for c in np.bincount(docs[b])]
    _run(synth.case_seed(9, 850), lens, lens, 2, 128, 128, "none", slope=-0.01)


@pytest.mark.parametrize("case", range(len(CASES)))
def test_varlen_backward(case):
    lq, lk, H, dqk, dv, kind, w, p, cap, slope = CASES[case]
    _run(synth.case_seed(9, 900 + case), lq, lk, H, dqk, dv, kind, w, p, cap, slope, backward=True)


def test_varlen_backward_without_queries():
    # total_q = 0 while the sequences hold keys: every dK / dV row is 0 (the buffers start
    # as NaN, so each must be written)
    import torch
    import block_sparse_attention_fmha_amd as fa
    dev = torch.device("cuda:0")
    _, k, v = synth.attention_inputs(synth.case_seed(9, 899), 1, 1, 300, 2, 128, 128, "bf16")
    tk, tv = (x.to_torch(dev)[0] for x in (k, v))
    none = torch.empty(0, 2, 128, device=dev, dtype=torch.bfloat16)
    cu_q = torch.tensor([0, 0, 0], dtype=torch.int32, device=dev)
    cu_k = torch.tensor([0, 100, 300], dtype=torch.int32, device=dev)
    lse = torch.empty(2, 0, device=dev, dtype=torch.float32)
    dk, dv = torch.full_like(tk, float("nan")), torch.full_like(tv, float("nan"))
    announce("varlen bwd total_q=0 total_k=300 H=2 D=128 causal")
    dq, dk, dv = fa.fmha_bwd_varlen(none, tk, tv, none, lse, none, cu_q, cu_k, 0, 200, mask=fa.Mask("causal"),
                                    dk=dk, dv=dv)
    torch.cuda.synchronize()
    assert dq.numel() == 0 and torch.all(dk == 0) and torch.all(dv == 0)
