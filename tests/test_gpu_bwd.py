"""GPU parity of the backward (dQ, dK, dV from the saved LSE) against the fp64 oracle,
and its determinism (no atomics: repeated runs are bitwise identical)."""
import numpy as np
import pytest

import oracle
from block_sparse_attention_fmha_amd import synth
from tests.gpu_util import announce, check_bf16, check_grad, host, mask_pair, to_dev

pytestmark = pytest.mark.gpu


def run_fwd_bwd(q, k, v, do, gmask=None, **kw):
    import torch
    import block_sparse_attention_fmha_amd as fa
    out, lse = fa.fmha_fwd(q, k, v, mask=gmask, **kw)
    dq, dk, dv = fa.fmha_bwd(q, k, v, out, lse, do, mask=gmask, **kw)
    torch.cuda.synchronize()
    return out, lse, dq, dk, dv


def _case(seed, B, Nq, Nk, H, Dqk, Dv, kind="none", window=0, prefix=0, softcap=0.0, slope=0.0,
          heads=None, lists=None):
    q, k, v, do = synth.attention_inputs(seed, B, Nq, Nk, H, Dqk, Dv, "bf16", with_dout=True)
    om, gm = mask_pair(kind, B, Nq, Nk, window, prefix, doc_seed=seed)
    announce(f"bwd bf16 seed={seed} B={B} Nq={Nq} Nk={Nk} H={H} D={Dqk}/{Dv} mask={kind} W={window} "
             f"P={prefix} softcap={softcap} bias={slope} lists={lists is not None}")
    kw = dict(softcap=softcap, bias_slope=slope)
    bs = None
    if lists is not None:
        import block_sparse_attention_fmha_amd as fa
        bs = fa.build_block_mask(gm, B, Nq, Nk, lists[0], lists[1])
    out, lse, dq, dk, dv = run_fwd_bwd(to_dev(q), to_dev(k), to_dev(v), to_dev(do), gm, block_sparse=bs, **kw)
    ref = oracle.backward(q.values, k.values, v.values, do.values, mask=om, heads=heads, **kw)
    hs = list(range(H)) if heads is None else heads
    for name, got, want in (("dQ", dq, ref[0]), ("dK", dk, ref[1]), ("dV", dv, ref[2])):
        check_grad(name, host(got)[:, :, hs], want[:, :, hs])
    check_bf16("O", host(out)[:, :, hs], ref[3][:, :, hs])
    check_bf16("LSE", host(lse)[:, hs], ref[4][:, hs])


SMALL = [
    (1, 256, 256, 2, 128, 128, "causal", 0, 0, 0.0, 0.0),
    (2, 256, 256, 2, 64, 64, "none", 0, 0, 0.0, 0.0),
    (1, 300, 300, 2, 128, 128, "causal", 0, 0, 0.0, 0.0),
    (1, 129, 257, 2, 128, 128, "causal", 0, 0, 0.0, 0.0),
    (1, 257, 129, 2, 128, 128, "causal", 0, 0, 0.0, 0.0),
    (1, 384, 384, 2, 192, 128, "causal", 0, 0, 0.0, 0.0),
    (1, 513, 769, 2, 128, 128, "sliding_window", 171, 0, 0.0, 0.0),
    (1, 512, 512, 2, 64, 64, "sliding_window", 100, 0, 30.0, 0.0),
    (2, 384, 384, 2, 128, 128, "prefix_lm", 0, 100, 0.0, -0.01),
    (2, 512, 512, 1, 128, 128, "block_diagonal", 0, 0, 0.0, -0.01),
    # odd lengths: row 1's document ids unaligned, ragged last tiles (vector and scalar loads)
    (2, 515, 517, 2, 128, 128, "block_diagonal", 0, 0, 0.0, 0.0),
    (2, 517, 515, 2, 64, 64, "block_diagonal", 0, 0, 0.0, 0.0),
    (1, 200, 200, 2, 128, 128, "none", 0, 0, 5.0, -0.05),
]


@pytest.mark.parametrize("case", range(len(SMALL)))
def test_bwd_small(case):
    B, Nq, Nk, H, Dqk, Dv, kind, W, P, cap, slope = SMALL[case]
    _case(synth.case_seed(9, 200 + case), B, Nq, Nk, H, Dqk, Dv, kind, W, P, cap, slope)


@pytest.mark.parametrize("kind", ["causal", "sliding_window", "block_diagonal", "prefix_lm"])
def test_bwd_block_sparse_lists(kind):
    _case(synth.case_seed(9, 300), 2, 1024, 1024, 2, 128, 128, kind, window=300, prefix=256,
          slope=-0.01, lists=(128, 128))


@pytest.mark.parametrize("kind", ["causal", "prefix_lm"])
def test_bwd_block_sparse_lists_mla(kind):
    # MLA-shaped heads (Dqk 192, Dv 128) through the transposed / forward lists
    _case(synth.case_seed(9, 310), 1, 1024, 1024, 2, 192, 128, kind, prefix=256, slope=-0.01,
          lists=(128, 128))


@pytest.mark.parametrize("kind", ["causal", "block_diagonal"])
def test_bwd_block_sparse_full_size(kind):
    # the block-sparse workload's shape (B=2 H=8 N=8192 D=128, 128x128 tiles, relative bias),
    # gradients compared on one head of both batch rows
    _case(synth.case_seed(9, 320), 2, 8192, 8192, 8, 128, 128, kind, slope=-0.01, heads=[3],
          lists=(128, 128))


@pytest.mark.parametrize("kind", ["none", "causal"])
def test_bwd_one_empty_side(kind):
    # no keys: every query's output is 0 and so is dQ; no queries: dK = dV = 0. The
    # gradient buffers start as NaN, so every element must be written.
    import torch
    import block_sparse_attention_fmha_amd as fa
    dev = torch.device("cuda:0")
    gm = fa.Mask(kind)
    q, k, v, do = (to_dev(x) for x in synth.attention_inputs(synth.case_seed(4, 90), 2, 300, 300, 3, 128, 128,
                                                               "bf16", with_dout=True))
    none = torch.empty(2, 0, 3, 128, device=dev, dtype=torch.bfloat16)
    announce(f"bwd Nk=0 B=2 Nq=300 H=3 D=128 mask={kind}")
    out, lse = fa.fmha_fwd(q, none, none, mask=gm)
    dq = torch.full_like(q, float("nan"))
    dq, dk, dv = fa.fmha_bwd(q, none, none, out, lse, do, mask=gm, dq=dq)
    torch.cuda.synchronize()
    assert torch.all(dq == 0) and dk.numel() == 0 and dv.numel() == 0
    lse0 = torch.empty(2, 3, 0, device=dev, dtype=torch.float32)
    announce(f"bwd Nq=0 B=2 Nk=300 H=3 D=128 mask={kind}")
    dk, dv = torch.full_like(k, float("nan")), torch.full_like(v, float("nan"))
    dq, dk, dv = fa.fmha_bwd(none, k, v, none, lse0, none, mask=gm, dk=dk, dv=dv)
    torch.cuda.synchronize()
    assert dq.numel() == 0 and torch.all(dk == 0) and torch.all(dv == 0)


def test_bwd_deterministic():
    import torch
    q, k, v, do = synth.attention_inputs(synth.case_seed(9, 400), 1, 1024, 1024, 4, 128, 128, "bf16",
                                         with_dout=True)
    tq, tk, tv, tdo = (to_dev(x) for x in (q, k, v, do))
    announce("bwd determinism B=1 N=1024 H=4 D=128 causal x3")
    _, gm = mask_pair("causal", 1, 1024, 1024)
    first = run_fwd_bwd(tq, tk, tv, tdo, gm)
    for _ in range(2):
        again = run_fwd_bwd(tq, tk, tv, tdo, gm)
        for a, b in zip(first, again):
            assert torch.equal(a, b)


CONFIG4 = [(4096, 64, 64), (4096, 128, 128), (16384, 64, 64), (16384, 128, 128), (8192, 192, 128)]


@pytest.mark.parametrize("case", range(len(CONFIG4)))
def test_bwd_full_size(case):
    N, Dqk, Dv = CONFIG4[case]
    _case(synth.case_seed(4, case), 1, N, N, 16, Dqk, Dv, "causal", heads=[case % 16])


def _random_list_cases(n=10, seed=2718):
    """Seeded block-sparse problems with arbitrary tile classes (not derived from a mask):
    (B, Nq, Nk, H, Hm, D, tile_m, tile_n, mask, class seed) per case."""
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        B = int(rng.integers(1, 4))
        H = int(rng.choice([2, 4]))
        Hm = int(rng.choice([1, H]))
        d = int(rng.choice([64, 128]))
        tm, tn = (int(x) for x in rng.choice([128, 256], 2))
        out.append((B, int(rng.integers(257, 1400)), int(rng.integers(257, 1400)), H, Hm, d, tm, tn,
                    str(rng.choice(["none", "causal"])), int(rng.integers(1 << 30))))
    return out


def _lists_from_classes(cls):
    """Forward and transposed lists of a class map cls [B, Hm, nQt, nKt] (0 skip, 1 partial,
    2 full), ascending and -1 padded, as numpy int32 arrays in BlockLists field order."""
    B, Hm, nqt, nkt = cls.shape

    def rows(c, n_rows, n_cols, val):
        cnt = np.zeros((B, Hm, n_rows), np.int32)
        idx = np.full((B, Hm, n_rows, n_cols), -1, np.int32)
        for b in range(B):
            for h in range(Hm):
                for r in range(n_rows):
                    sel = np.nonzero(c[b, h, r] == val)[0]
                    cnt[b, h, r] = len(sel)
                    idx[b, h, r, :len(sel)] = sel
        return cnt, idx

    pc, pi = rows(cls, nqt, nkt, 1)
    fc, fi = rows(cls, nqt, nkt, 2)
    t = np.ascontiguousarray(cls.transpose(0, 1, 3, 2))
    tpc, tpi = rows(t, nkt, nqt, 1)
    tfc, tfi = rows(t, nkt, nqt, 2)
    return pc, pi, fc, fi, tpc, tpi, tfc, tfi


@pytest.mark.parametrize("case", range(10))
def test_bwd_random_lists(case):
    # arbitrary per-head lists over several batch rows: the workgroups take their tiles in
    # order of list length (per batch row and mask head), rows and key tiles without any
    # listed tile give O = 0 / LSE = -inf / dQ = 0 and dK = dV = 0
    import torch
    import block_sparse_attention_fmha_amd as fa
    B, Nq, Nk, H, Hm, d, tm, tn, kind, cseed = _random_list_cases()[case]
    nqt, nkt = -(-Nq // tm), -(-Nk // tn)
    rng = np.random.default_rng(cseed)
    cls = rng.integers(0, 3, size=(B, Hm, nqt, nkt))
    cls[0, 0, nqt - 1] = 0          # an empty query-tile row
    cls[B - 1, Hm - 1, :, 0] = 0     # an empty key-tile column
    arrays = _lists_from_classes(cls)
    seed = synth.case_seed(9, 700 + case)
    q, k, v, do = synth.attention_inputs(seed, B, Nq, Nk, H, d, d, "bf16", with_dout=True)
    om, gm = mask_pair(kind, B, Nq, Nk)
    announce(f"bwd random lists case={case} B={B} Nq={Nq} Nk={Nk} H={H} Hm={Hm} D={d} tiles={tm}x{tn} mask={kind}")
    dev = torch.device("cuda:0")
    bs = fa.BlockSparse(tm, tn, nqt, nkt, Hm, *(torch.from_numpy(a).to(dev) for a in arrays))
    out, lse, dq, dk, dv = run_fwd_bwd(to_dev(q), to_dev(k), to_dev(v), to_dev(do), gm, block_sparse=bs)
    lists = oracle.BlockLists(tm, tn, *arrays)
    ref = oracle.backward(q.values, k.values, v.values, do.values, mask=om, lists=lists)
    for name, got, want in (("dQ", dq, ref[0]), ("dK", dk, ref[1]), ("dV", dv, ref[2])):
        check_grad(name, host(got), want)
    check_bf16("O", host(out), ref[3])
    check_bf16("LSE", host(lse), ref[4])
