"""GPU tests with tensors larger than 4 GiB: every Q / K / V / O / gradient tensor of the
prefill cases is 4.5 GiB (the decode case reads an 8 GiB K / V cache), so the sampled batches sit past the signed (2 GiB) and unsigned (4 GiB) 32-bit
byte offsets. Inputs: the seeded causal N=16384 D=128 H=16 block, with batch b holding it
rolled by 97 b along the sequence and by b along the heads (every batch distinct, so an
offset that wrapped would read another batch's values).

Forward: sampled rows of far batches against the fp64 oracle. Backward: the gradients of
a far batch must equal, bit for bit, those of a one-batch launch on a copy of that batch
(the kernels are deterministic and a (batch, head) never depends on the others); the
one-batch backward itself is held to the oracle by the other backward tests."""
import numpy as np
import pytest

import oracle
from block_sparse_attention_fmha_amd import synth
from tests.gpu_util import announce, check_bf16, device, host, mask_pair

pytestmark = pytest.mark.gpu

B, N, H, D = 72, 16384, 16, 128
FAR = (71, 40)   # byte offsets 4.4 GiB and 2.5 GiB into each tensor


def _shift(b):
    return (97 * b) % N, b % H


@pytest.fixture(scope="module")
def big():
    import torch
    seed = synth.case_seed(11, 0)
    q, k, v, do = synth.attention_inputs(seed, 1, N, N, H, D, D, "bf16", with_dout=True)
    dev = device()
    announce(f"large tensors seed={seed} B={B} N={N} H={H} D={D} (4.5 GiB each)")
    out = []
    for t in (q, k, v, do):
        base = t.to_torch(dev)[0]
        x = torch.empty((B, N, H, D), dtype=base.dtype, device=dev)
        for b in range(B):
            x[b].copy_(torch.roll(base, shifts=_shift(b), dims=(0, 1)))
        out.append(x)
    torch.cuda.synchronize()
    return (q, k, v, do), out


def _host_batch(t, b):
    return np.roll(t.values[0], _shift(b), axis=(0, 1))


def test_fwd_beyond_4gib(big):
    import torch
    import block_sparse_attention_fmha_amd as fa
    (q, k, v, _), (tq, tk, tv, _) = big
    om, gm = mask_pair("causal", 1, N, N)
    announce(f"fwd causal B={B} N={N} H={H} D={D} beyond 4 GiB")
    out, lse = fa.fmha_fwd(tq, tk, tv, mask=gm)
    torch.cuda.synchronize()
    rng = np.random.default_rng(7)
    rows = np.unique(np.concatenate([np.arange(64), np.arange(N - 64, N), rng.integers(0, N, 64)]))
    ridx = torch.from_numpy(rows).to(out.device)
    for b in FAR:
        qb, kb, vb = (_host_batch(t, b) for t in (q, k, v))
        for h in (H - 1, 3):
            o_ref, l_ref = oracle.forward_bh(qb[rows, h], kb[:, h], vb[:, h], rows, 0, h, N, N,
                                             scale=1 / np.sqrt(D), mask=om)
            check_bf16(f"O[{b},{h}]", host(out[b, :, h].index_select(0, ridx)), o_ref)
            check_bf16(f"LSE[{b},{h}]", host(lse[b, h].index_select(0, ridx)), l_ref)


def test_bwd_beyond_4gib_equals_one_batch(big):
    import torch
    import block_sparse_attention_fmha_amd as fa
    _, (tq, tk, tv, tdo) = big
    gm = mask_pair("causal", 1, N, N)[1]
    announce(f"bwd causal B={B} N={N} H={H} D={D} beyond 4 GiB")
    out, lse = fa.fmha_fwd(tq, tk, tv, mask=gm)
    dq, dk, dv = fa.fmha_bwd(tq, tk, tv, out, lse, tdo, mask=gm)
    torch.cuda.synchronize()
    for b in FAR:
        announce(f"bwd one-batch copy of batch {b}")
        q1, k1, v1, do1 = (t[b:b + 1].clone() for t in (tq, tk, tv, tdo))
        o1, l1 = fa.fmha_fwd(q1, k1, v1, mask=gm)
        g1 = fa.fmha_bwd(q1, k1, v1, o1, l1, do1, mask=gm)
        torch.cuda.synchronize()
        assert torch.equal(out[b:b + 1], o1), f"O of batch {b} differs from its one-batch launch"
        assert torch.equal(lse[b:b + 1], l1), f"LSE of batch {b} differs from its one-batch launch"
        for name, big_g, one_g in (("dQ", dq, g1[0]), ("dK", dk, g1[1]), ("dV", dv, g1[2])):
            assert torch.equal(big_g[b:b + 1], one_g), f"{name} of batch {b} differs from its one-batch launch"


def test_splitkv_beyond_4gib():
    # decode over an 8 GiB K / V cache: B=4 H=8 Nq=1 Nk=2^20 D=128, 16 splits. Key block j
    # (16384 keys) of batch b is the seeded block rolled by 97 (64 b + j) along the keys and
    # by b + j along the heads; sampled (b, h) rows against the fp64 oracle
    import torch
    import block_sparse_attention_fmha_amd as fa
    Bd, Hd, NB = 4, 8, 64
    Nk = NB * N
    seed = synth.case_seed(11, 1)
    q = synth.attention_inputs(seed, Bd, 1, 1, Hd, D, D, "bf16")[0]
    _, k0, v0 = synth.attention_inputs(seed + 1, 1, 1, N, Hd, D, D, "bf16")
    dev = device()
    announce(f"splitkv seed={seed} B={Bd} H={Hd} Nk={Nk} D={D} beyond 4 GiB")

    def shift(b, j):
        return (97 * (NB * b + j)) % N, (b + j) % Hd

    kv = []
    for t in (k0, v0):
        base = t.to_torch(dev)[0]
        x = torch.empty((Bd, Nk, Hd, D), dtype=base.dtype, device=dev)
        for b in range(Bd):
            for j in range(NB):
                x[b, j * N:(j + 1) * N].copy_(torch.roll(base, shifts=shift(b, j), dims=(0, 1)))
        kv.append(x)
    out, lse = fa.fmha_fwd_splitkv(q.to_torch(dev), kv[0], kv[1], 16)
    torch.cuda.synchronize()
    o, l = host(out), host(lse)
    for b, h in ((3, 7), (2, 0)):
        kh = np.concatenate([np.roll(k0.values[0], shift(b, j), axis=(0, 1))[:, h] for j in range(NB)])
        vh = np.concatenate([np.roll(v0.values[0], shift(b, j), axis=(0, 1))[:, h] for j in range(NB)])
        o_ref, l_ref = oracle.forward_bh(q.values[b, :, h], kh, vh, np.arange(1), b, h, 1, Nk,
                                         scale=1 / np.sqrt(D))
        check_bf16(f"O[{b},{h}]", o[b, :, h], o_ref)
        check_bf16(f"LSE[{b},{h}]", l[b, h], l_ref)
