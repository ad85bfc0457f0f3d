"""GPU block-mask builder (bit-exact against the oracle's element enumeration) and the
block-sparse forward driven by its lists."""
import numpy as np
import pytest

import oracle
from block_sparse_attention_fmha_amd import synth
from tests.gpu_util import announce, check_bf16, host, mask_pair, to_dev

pytestmark = pytest.mark.gpu

FIELDS = ("partial_cnt", "partial_idx", "full_cnt", "full_idx", "t_partial_cnt", "t_partial_idx",
          "t_full_cnt", "t_full_idx")


def _build(gm, B, Nq, Nk, tm, tn):
    import torch
    import block_sparse_attention_fmha_amd as fa
    bs = fa.build_block_mask(gm, B, Nq, Nk, tm, tn)
    torch.cuda.synchronize()
    return bs


@pytest.mark.parametrize("kind,W,P", [("none", 0, 0), ("causal", 0, 0), ("sliding_window", 2730, 0),
                                      ("prefix_lm", 0, 1024), ("block_diagonal", 0, 0)])
@pytest.mark.parametrize("B,Nq,Nk,tm,tn", [(2, 8192, 8192, 128, 128), (1, 1000, 1300, 128, 64),
                                           (2, 777, 555, 100, 37)])
def test_block_lists_bit_exact(kind, W, P, B, Nq, Nk, tm, tn):
    seed = synth.case_seed(3, 0)
    om, gm = mask_pair(kind, B, Nq, Nk, W, P, doc_seed=seed)
    announce(f"build_block_mask {kind} B={B} Nq={Nq} Nk={Nk} tile={tm}x{tn}")
    bs = _build(gm, B, Nq, Nk, tm, tn)
    ref = oracle.build_lists(om, B, 1, Nq, Nk, tm, tn)
    for f in FIELDS:
        got = getattr(bs, f).cpu().numpy()
        assert np.array_equal(got, getattr(ref, f)), f


BS_CASES = [("causal", 0, 0), ("sliding_window", 2730, 0), ("block_diagonal", 0, 0), ("prefix_lm", 0, 1024)]


@pytest.mark.parametrize("kind,W,P", BS_CASES)
def test_block_sparse_forward_full_size(kind, W, P):
    # B=2 H=8 N=8192 D=128, 128x128 tiles, relative bias -0.01|i-j|; heads 0 and 5 of
    # both batch rows compared on sampled rows
    seed = synth.case_seed(3, BS_CASES.index((kind, W, P)))
    B, N, H, D = 2, 8192, 8, 128
    q, k, v = synth.attention_inputs(seed, B, N, N, H, D, D, "bf16")
    om, gm = mask_pair(kind, B, N, N, W, P, doc_seed=seed)
    announce(f"block-sparse fwd {kind} seed={seed} B=2 N=8192 H=8 D=128")
    import torch
    import block_sparse_attention_fmha_amd as fa
    bs = _build(gm, B, N, N, 128, 128)
    out, lse = fa.fmha_fwd(to_dev(q), to_dev(k), to_dev(v), mask=gm, block_sparse=bs, bias_slope=-0.01)
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([np.arange(0, 200), np.arange(N - 200, N),
                                     np.random.default_rng(seed).choice(N, 300, replace=False)]))
    heads = [0, 5]
    o_ref, l_ref = oracle.forward(q.values, k.values, v.values, mask=om, bias_slope=-0.01, rows=rows, heads=heads)
    o, l = host(out), host(lse)
    check_bf16("O", o[:, rows][:, :, heads], o_ref[:, rows][:, :, heads])
    check_bf16("LSE", l[:, heads][:, :, rows], l_ref[:, heads][:, :, rows])


def test_block_sparse_custom_lists_small():
    # arbitrary lists (not derived from the mask): full tiles ignore the element mask,
    # partial tiles apply it, unlisted tiles are skipped
    import torch
    import block_sparse_attention_fmha_amd as fa
    B, N, H, D, T = 1, 512, 2, 128, 128
    q, k, v = synth.attention_inputs(synth.case_seed(9, 600), B, N, N, H, D, D, "bf16")
    nt = N // T
    rng = np.random.default_rng(5)
    cls = rng.integers(0, 3, size=(nt, nt))   # 0 skip, 1 partial, 2 full
    lists = {}
    pc = np.zeros((1, 1, nt), np.int32); pi = np.full((1, 1, nt, nt), -1, np.int32)
    fc = np.zeros((1, 1, nt), np.int32); fi = np.full((1, 1, nt, nt), -1, np.int32)
    for r in range(nt):
        p = np.nonzero(cls[r] == 1)[0]; f = np.nonzero(cls[r] == 2)[0]
        pc[0, 0, r] = len(p); pi[0, 0, r, :len(p)] = p
        fc[0, 0, r] = len(f); fi[0, 0, r, :len(f)] = f
    dev = torch.device("cuda:0")
    t = lambda a: torch.from_numpy(a).to(dev)
    bs = fa.BlockSparse(T, T, nt, nt, 1, t(pc), t(pi), t(fc), t(fi), None, None, None, None)
    om, gm = mask_pair("causal", B, N, N)
    announce("block-sparse fwd with custom lists N=512")
    out, lse = fa.fmha_fwd(to_dev(q), to_dev(k), to_dev(v), mask=gm, block_sparse=bs)
    torch.cuda.synchronize()
    ref_lists = oracle.BlockLists(T, T, pc, pi, fc, fi, None, None, None, None)
    o_ref, l_ref = oracle.forward(q.values, k.values, v.values, mask=om, lists=ref_lists)
    check_bf16("O", host(out), o_ref)
    check_bf16("LSE", host(lse), l_ref)
