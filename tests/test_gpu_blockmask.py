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


def _label_runs(rng, B, N, nlab):
    """Runs of 50..3000 tokens, each labelled from nlab labels at random: a label recurs in
    runs that are not adjacent, so one 'document' spans separate ranges."""
    out = np.empty((B, N), dtype=np.int32)
    for b in range(B):
        pos = 0
        while pos < N:
            end = min(N, pos + int(rng.integers(50, 3000, endpoint=True)))
            out[b, pos:end] = rng.integers(0, nlab)
            pos = end
    return out


@pytest.mark.parametrize("B,Nq,Nk,tm,tn,ndoc", [(1, 9000, 7500, 1500, 1100, 3), (2, 5000, 6000, 64, 128, 4),
                                                (1, 12300, 8197, 2050, 1025, 2)])
def test_block_lists_unsorted_documents(B, Nq, Nk, tm, tn, ndoc):
    # document ids that are not sorted (a label recurs in separate runs), and tiles wider
    # than the builder's 1024-id LDS chunk
    import torch
    import block_sparse_attention_fmha_amd as fa
    rng = np.random.default_rng(synth.case_seed(3, 50 + ndoc))
    dq, dk = _label_runs(rng, B, Nq, ndoc), _label_runs(rng, B, Nk, ndoc)
    om = oracle.MaskSpec("block_diagonal", doc_q=dq, doc_k=dk)
    dev = torch.device("cuda:0")
    gm = fa.Mask("block_diagonal", doc_q=torch.from_numpy(dq).to(dev), doc_k=torch.from_numpy(dk).to(dev))
    announce(f"build_block_mask unsorted docs B={B} Nq={Nq} Nk={Nk} tile={tm}x{tn} ndoc={ndoc}")
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


@pytest.mark.parametrize("N,TM,TN,heads,kind", [(512, 128, 128, 1, "causal"), (700, 128, 192, 2, "causal"),
                                               (1100, 384, 64, 2, "causal"), (300, 256, 128, 1, "causal"),
                                               (1100, 128, 128, 2, "none"), (2000, 256, 64, 2, "none")])
def test_block_sparse_custom_lists_small(N, TM, TN, heads, kind):
    # arbitrary lists (not derived from the mask): full tiles ignore the element mask,
    # partial tiles apply it, unlisted tiles are skipped. Entries are unsorted, some are
    # repeated, some columns sit in both lists of a row (full wins), and one row is empty
    # (its queries see nothing: O = 0, LSE = -inf). Without a band mask ("none") the
    # workgroups take their query tiles in order of list length, per head.
    import torch
    import block_sparse_attention_fmha_amd as fa
    B, H, D = 1, 2, 128
    q, k, v = synth.attention_inputs(synth.case_seed(9, 600 + N), B, N, N, H, D, D, "bf16")
    nqt, nkt = -(-N // TM), -(-N // TN)
    rng = np.random.default_rng(N + TM + TN)
    pc = np.zeros((B, heads, nqt), np.int32); pi = np.full((B, heads, nqt, nkt), -1, np.int32)
    fc = np.zeros((B, heads, nqt), np.int32); fi = np.full((B, heads, nqt, nkt), -1, np.int32)
    for hh in range(heads):
        cls = rng.integers(0, 3, size=(nqt, nkt))   # 0 skip, 1 partial, 2 full
        cls[nqt - 1] = 0 if nqt > 1 else cls[nqt - 1]
        for r in range(nqt):
            p = list(rng.permutation(np.nonzero(cls[r] == 1)[0]))
            f = list(rng.permutation(np.nonzero(cls[r] == 2)[0]))
            if len(p) > 1 and len(p) < nkt:
                p.append(p[0])                    # repeated entry
            if len(f) and len(p) < nkt:
                p.append(f[-1])                   # also listed as full
            pc[0, hh, r] = len(p); pi[0, hh, r, :len(p)] = p
            fc[0, hh, r] = len(f); fi[0, hh, r, :len(f)] = f
    dev = torch.device("cuda:0")
    t = lambda a: torch.from_numpy(a).to(dev)
    bs = fa.BlockSparse(TM, TN, nqt, nkt, heads, t(pc), t(pi), t(fc), t(fi), None, None, None, None)
    om, gm = mask_pair(kind, B, N, N)
    announce(f"block-sparse fwd with custom lists N={N} tiles={TM}x{TN} heads={heads} mask={kind}")
    out, lse = fa.fmha_fwd(to_dev(q), to_dev(k), to_dev(v), mask=gm, block_sparse=bs)
    torch.cuda.synchronize()
    ref_lists = oracle.BlockLists(TM, TN, pc, pi, fc, fi, None, None, None, None)
    o_ref, l_ref = oracle.forward(q.values, k.values, v.values, mask=om, lists=ref_lists)
    check_bf16("O", host(out), o_ref)
    check_bf16("LSE", host(lse), l_ref)


@pytest.mark.parametrize("kind,tm", [("causal", 128), ("causal", 256), ("sliding_window", 128),
                                     ("prefix_lm", 256), ("none", 128)])
def test_lists_from_mask_match_analytic_ranges_bitwise(kind, tm):
    # lists built from a band mask visit the same 64-key tiles in the same ascending order as
    # the analytic ranges, masking exactly where the analytic path masks, so the forward (O,
    # LSE) and the backward (dQ, dK, dV) come out bitwise equal; N = 1000 leaves a ragged
    # last tile on both sides. (The analytic forward runs unsplit: this short grid would
    # otherwise take the key split, whose combine rounds differently.)
    import torch
    import block_sparse_attention_fmha_amd as fa
    B, N, H, D = 2, 1000, 2, 128
    q, k, v, do = (to_dev(x) for x in synth.attention_inputs(synth.case_seed(9, 650), B, N, N, H, D, D, "bf16",
                                                             with_dout=True))
    m = fa.Mask(kind, window=300, prefix=200)
    announce(f"lists vs analytic ranges, bitwise: mask={kind} tile_m={tm} B={B} N={N} H={H}")
    bs = fa.build_block_mask(m, B, N, N, tm, 128)
    for slope in (0.0, -0.01):
        o1, l1 = fa.fmha_fwd(q, k, v, mask=m, bias_slope=slope, key_split=False)
        o2, l2 = fa.fmha_fwd(q, k, v, mask=m, bias_slope=slope, block_sparse=bs)
        g1 = fa.fmha_bwd(q, k, v, o1, l1, do, mask=m, bias_slope=slope)
        g2 = fa.fmha_bwd(q, k, v, o2, l2, do, mask=m, bias_slope=slope, block_sparse=bs)
        torch.cuda.synchronize()
        assert torch.equal(o1, o2) and torch.equal(l1, l2), f"forward differs (bias {slope})"
        for name, a, b in zip(("dQ", "dK", "dV"), g1, g2):
            assert torch.equal(a, b), f"{name} differs (bias {slope})"
