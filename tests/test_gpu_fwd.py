"""GPU parity of the forward (bf16 and fp32) against the fp64 oracle.

Small cases compare every output element; the full-size workloads compare sampled
heads / rows that the oracle computes one by one (the oracle is exact per row, so a
sampled row is as strict as a full comparison of that row)."""
import functools

import numpy as np
import pytest

import oracle
from block_sparse_attention_fmha_amd import synth
from tests.gpu_util import (announce, check_bf16, check_fp32, device, host, mask_pair, to_dev)

pytestmark = pytest.mark.gpu


def run_fwd(q, k, v, gmask=None, **kw):
    import block_sparse_attention_fmha_amd as fa
    out, lse = fa.fmha_fwd(q, k, v, mask=gmask, **kw)
    import torch
    torch.cuda.synchronize()
    return out, lse


def _case(seed, B, Nq, Nk, H, Dqk, Dv, dtype, kind="none", window=0, prefix=0, softcap=0.0,
          slope=0.0, rows=None, heads=None):
    q, k, v = synth.attention_inputs(seed, B, Nq, Nk, H, Dqk, Dv, dtype)
    om, gm = mask_pair(kind, B, Nq, Nk, window, prefix, doc_seed=seed)
    announce(f"fwd {dtype} seed={seed} B={B} Nq={Nq} Nk={Nk} H={H} D={Dqk}/{Dv} mask={kind} "
             f"W={window} P={prefix} softcap={softcap} bias={slope}")
    out, lse = run_fwd(to_dev(q), to_dev(k), to_dev(v), gm, softcap=softcap, bias_slope=slope)
    o_ref, l_ref = oracle.forward(q.values, k.values, v.values, softcap=softcap, bias_slope=slope,
                                  mask=om, rows=rows, heads=heads)
    o, l = host(out), host(lse)
    rsel = slice(None) if rows is None else np.asarray(rows)
    hsel = slice(None) if heads is None else np.asarray(heads)
    if dtype == "fp32":
        check_fp32("O", o[:, rsel][:, :, hsel], o_ref[:, rsel][:, :, hsel])
        check_fp32("LSE", l[:, hsel][:, :, rsel], l_ref[:, hsel][:, :, rsel])
    else:
        check_bf16("O", o[:, rsel][:, :, hsel], o_ref[:, rsel][:, :, hsel])
        check_bf16("LSE", l[:, hsel][:, :, rsel], l_ref[:, hsel][:, :, rsel])


# ------------------------------------------------------------------ small, every element

SMALL = [
    # (B, Nq, Nk, H, Dqk, Dv, kind, window, prefix, softcap, slope)
    (2, 256, 256, 3, 128, 128, "none", 0, 0, 0.0, 0.0),
    (2, 256, 256, 3, 128, 128, "causal", 0, 0, 0.0, 0.0),
    (1, 300, 300, 2, 128, 128, "causal", 0, 0, 0.0, 0.0),
    (1, 129, 257, 2, 128, 128, "causal", 0, 0, 0.0, 0.0),
    (1, 257, 129, 2, 128, 128, "causal", 0, 0, 0.0, 0.0),      # rows with no visible key
    (1, 513, 769, 2, 128, 128, "sliding_window", 171, 0, 0.0, 0.0),
    (1, 640, 640, 2, 64, 64, "sliding_window", 100, 0, 30.0, 0.0),
    (2, 384, 384, 2, 64, 64, "prefix_lm", 0, 100, 0.0, -0.01),
    (2, 512, 512, 2, 128, 128, "block_diagonal", 0, 0, 0.0, -0.01),
    # odd lengths: batch row 1's document ids are not 16-byte aligned and the last key tile
    # is ragged, so both the vector and the scalar document loads run
    (2, 515, 517, 2, 128, 128, "block_diagonal", 0, 0, 0.0, 0.0),
    (2, 517, 515, 2, 64, 64, "block_diagonal", 0, 0, 0.0, 0.0),
    (1, 255, 385, 2, 192, 128, "causal", 0, 0, 0.0, 0.0),      # MLA-shaped heads
    (1, 200, 200, 2, 128, 128, "none", 0, 0, 5.0, -0.05),
    (1, 300, 300, 2, 128, 128, "causal", 0, 0, 30.0, 0.0),     # softcap, fixed softmax maximum
    (1, 300, 300, 2, 128, 128, "none", 0, 0, 50.0, 0.0),       # softcap above that path's limit
    (1, 1, 1000, 4, 128, 128, "causal", 0, 0, 0.0, 0.0),       # single decode query
    (1, 1000, 1, 2, 64, 64, "none", 0, 0, 0.0, 0.0),
]


@pytest.mark.parametrize("case", range(len(SMALL)))
def test_fwd_bf16_small(case):
    B, Nq, Nk, H, Dqk, Dv, kind, W, P, cap, slope = SMALL[case]
    _case(synth.case_seed(9, case), B, Nq, Nk, H, Dqk, Dv, "bf16", kind, W, P, cap, slope)


def test_fwd_bf16_softcap_saturated_rows():
    """Softcap 30 with every score far below -30 before the cap: each row's capped scores
    all sit near -30, so every probability is near 2^-86.6 relative to the cap, the
    smallest the fixed-maximum softmax produces; O must still be the visible keys'
    weighted mean (nearly the plain mean of V)."""
    q, k, v = synth.attention_inputs(synth.case_seed(9, 60), 1, 200, 200, 2, 128, 128, "bf16")
    def shifted(t, shift):
        x = np.float32(shift) + np.float32(0.25) * t.values
        bits = synth.bf16_bits(x)
        return synth.Tensor(synth.bf16_bits_to_f32(bits), bits, "bf16")
    q, k = shifted(q, 4.0), shifted(k, -4.0)      # raw scores near -128 * 16 = -2048
    for kind in ("none", "causal"):
        om, gm = mask_pair(kind, 1, 200, 200)
        announce(f"fwd bf16 softcap 30 saturated mask={kind}")
        out, lse = run_fwd(to_dev(q), to_dev(k), to_dev(v), gm, softcap=30.0)
        o_ref, l_ref = oracle.forward(q.values, k.values, v.values, softcap=30.0, mask=om)
        check_bf16("O", host(out), o_ref)
        check_bf16("LSE", host(lse), l_ref)


def test_fwd_bf16_empty_keys_and_queries():
    import torch
    import block_sparse_attention_fmha_amd as fa
    dev = device()
    q = torch.randn(1, 70, 2, 128, device=dev).bfloat16()
    k = torch.empty(1, 0, 2, 128, device=dev, dtype=torch.bfloat16)
    announce("fwd bf16 Nk=0")
    out, lse = run_fwd(q, k, k)
    assert torch.all(out == 0) and torch.all(torch.isneginf(lse))
    announce("fwd bf16 Nq=0")
    q0 = torch.empty(1, 0, 2, 128, device=dev, dtype=torch.bfloat16)
    kk = torch.randn(1, 5, 2, 128, device=dev).bfloat16()
    out, lse = run_fwd(q0, kk, kk)
    assert out.shape == (1, 0, 2, 128)


def test_fwd_bf16_strided_bhsd_layout():
    # BHSD storage passed as BSHD views: only the strides differ
    q, k, v = synth.attention_inputs(synth.case_seed(9, 50), 2, 200, 200, 3, 128, 128, "bf16")
    qt, kt, vt = (to_dev(x).permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3) for x in (q, k, v))
    assert qt.stride(2) == 200 * 128
    announce("fwd bf16 strided BHSD B=2 N=200 H=3")
    out, lse = run_fwd(qt, kt, vt, mask_pair("causal", 2, 200, 200)[1])
    o_ref, l_ref = oracle.forward(q.values, k.values, v.values, mask=oracle.MaskSpec("causal"))
    check_bf16("O", host(out), o_ref)
    check_bf16("LSE", host(lse), l_ref)


FP32_SMALL = [
    # (B, Nq, Nk, H, D, kind, prefix)
    (1, 128, 128, 1, 64, "causal", 0),      # the fp32 parity workload
    (2, 150, 170, 2, 64, "none", 0),
    (1, 200, 200, 2, 128, "sliding_window", 0),
    (1, 100, 130, 2, 1024, "causal", 0),
    (1, 600, 600, 1, 64, "block_diagonal", 0),
    (1, 130, 160, 2, 128, "prefix_lm", 70),
    (1, 90, 90, 2, 1024, "prefix_lm", 40),
]


@pytest.mark.parametrize("case", range(len(FP32_SMALL)))
def test_fwd_fp32_small(case):
    B, Nq, Nk, H, D, kind, prefix = FP32_SMALL[case]
    seed = synth.case_seed(1, 0) if case == 0 else synth.case_seed(9, 100 + case)
    _case(seed, B, Nq, Nk, H, D, D, "fp32", kind, window=50, prefix=prefix)


# (case index for the seed, B, N, H, D): seeds whose documents split every batch row
# (two rows of 637 + 263 and 261 + 500 + 139 tokens; one row of 435 + 335 + 230 and of
# 435 + 335 + 30), so keys of other documents sit inside every query tile's walk
FP32_DOCS = [(306, 2, 900, 2, 64), (309, 1, 1000, 2, 128), (309, 1, 800, 1, 1024)]


@pytest.mark.parametrize("case", range(len(FP32_DOCS)))
def test_fwd_fp32_block_diagonal_documents(case):
    c, B, N, H, D = FP32_DOCS[case]
    seed = synth.case_seed(9, c)
    assert all(len(np.unique(row)) >= 2 for row in synth.document_ids(seed, B, N))
    _case(seed, B, N, N, H, D, D, "fp32", "block_diagonal")


# ------------------------------------------------------------------ full-size workloads

def _rows_sample(n, seed):
    rng = np.random.default_rng(seed)
    pick = np.concatenate([np.arange(min(n, 64)), np.arange(max(0, n - 64), n),
                           rng.choice(n, size=min(n, 256), replace=False)])
    return np.unique(pick)


CONFIG2 = [(n, d, kind, cap) for n in (1024, 4096, 16384) for d in (64, 128)
           for kind in ("none", "causal", "sliding_window") for cap in (0.0, 30.0)]


@pytest.mark.parametrize("case", range(len(CONFIG2)))
def test_fwd_bf16_full_size(case):
    N, D, kind, cap = CONFIG2[case]
    seed = synth.case_seed(2, case)
    heads = None if N <= 1024 else [case % 16]
    rows = _rows_sample(N, seed) if N >= 16384 else None
    _case(seed, 1, N, N, 16, D, D, "bf16", kind, window=1024, softcap=cap, rows=rows, heads=heads)


def test_fwd_fp32_wide_head_full_size():
    # B=4 H=8 N=512 D=1024, no mask; two (b, h) pairs compared in full
    seed = synth.case_seed(5, 1)
    q, k, v = synth.attention_inputs(seed, 4, 512, 512, 8, 1024, 1024, "fp32")
    announce(f"fwd fp32 wide head seed={seed} B=4 N=512 H=8 D=1024")
    out, lse = run_fwd(to_dev(q), to_dev(k), to_dev(v))
    o, l = host(out), host(lse)
    for b, h in ((0, 0), (3, 5)):
        o_ref, l_ref = oracle.forward_bh(q.values[b, :, h], k.values[b, :, h], v.values[b, :, h],
                                         np.arange(512), b, h, 512, 512, scale=1 / 32.0)
        check_fp32(f"O[{b},{h}]", o[b, :, h], o_ref)
        check_fp32(f"LSE[{b},{h}]", l[b, h], l_ref)


# ------------------------------------------------------------------ key-split forward

KEY_SPLIT = [
    # (B, Nq, Nk, H, Hkv, D, kind, window, prefix, softcap, slope): short query sides against
    # long key ranges, so that the forward splits the keys
    (1, 256, 8192, 16, 16, 128, "none", 0, 0, 0.0, 0.0),
    (1, 256, 8192, 16, 16, 128, "causal", 0, 0, 0.0, 0.0),
    (1, 256, 8192, 16, 16, 128, "sliding_window", 3000, 0, 0.0, 0.0),   # 51 tiles in 7 parts
    (1, 256, 8192, 16, 16, 128, "prefix_lm", 0, 200, 30.0, 0.0),
    (1, 256, 8192, 16, 16, 64, "causal", 0, 0, 0.0, -0.01),
    (1, 256, 8192, 16, 4, 128, "causal", 0, 0, 0.0, 0.0),       # grouped K/V heads
    (2, 300, 5000, 3, 3, 128, "none", 0, 0, 0.0, 0.0),          # ragged rows and keys
    (1, 129, 8000, 2, 2, 64, "causal", 0, 0, 0.0, 0.0),         # 16 parts of a ragged range
    # causal imbalance and small grids: split and unsplit query tiles in one launch
    (1, 2048, 2048, 16, 16, 128, "causal", 0, 0, 0.0, 0.0),     # 1-3 parts of up to 12 tiles
    (1, 4096, 4096, 2, 2, 128, "causal", 0, 0, 0.0, 0.0),       # up to 8 parts of 8 tiles
    (1, 2000, 2000, 4, 4, 64, "prefix_lm", 0, 300, 0.0, 0.0),   # ragged last query tile
    (1, 700, 3000, 4, 4, 128, "causal", 0, 0, 30.0, -0.02),     # Nq < Nk: 5-6 parts, softcap + bias
    (1, 512, 4096, 4, 4, 128, "sliding_window", 1500, 0, 0.0, 0.0),  # window: 4 parts of 7
]


@pytest.mark.parametrize("case", range(len(KEY_SPLIT)))
def test_fwd_bf16_key_split(case):
    import block_sparse_attention_fmha_amd as fa
    B, Nq, Nk, H, Hkv, D, kind, W, P, cap, slope = KEY_SPLIT[case]
    seed = synth.case_seed(9, 300 + case)
    q, k, v = synth.normal_tensors(seed, [(B, Nq, H, D), (B, Nk, Hkv, D), (B, Nk, Hkv, D)], "bf16")
    om, gm = mask_pair(kind, B, Nq, Nk, W, P)
    tq, tk, tv = to_dev(q), to_dev(k), to_dev(v)
    assert fa.fwd_workspace_size(tq, tk, tv, mask=gm) > 0, "the case should take the key-split path"
    heads = None if H <= 4 else [0, 7, H - 1]
    o_ref, l_ref = oracle.forward(q.values, k.values, v.values, softcap=cap, bias_slope=slope, mask=om, heads=heads)
    hsel = slice(None) if heads is None else np.asarray(heads)
    for split in (True, False):
        announce(f"fwd bf16 key_split={split} B={B} Nq={Nq} Nk={Nk} H={H} Hkv={Hkv} D={D} mask={kind} "
                 f"softcap={cap} bias={slope}")
        out, lse = fa.fmha_fwd(tq, tk, tv, mask=gm, softcap=cap, bias_slope=slope, key_split=split)
        import torch
        torch.cuda.synchronize()
        check_bf16(f"O split={split}", host(out)[:, :, hsel], o_ref[:, :, hsel])
        check_bf16(f"LSE split={split}", host(lse)[:, hsel], l_ref[:, hsel])


@functools.lru_cache(maxsize=1)
def _key_split_fuzz_cases(n=16, seed=4242):
    """Seeded random forwards that take the key-split path: (B, Nq, Nk, H, Hkv, D, kind,
    window, prefix, softcap, slope), drawn until n of them split (checked with the
    library's own workspace query on empty tensors of those shapes)."""
    import random
    import torch
    import block_sparse_attention_fmha_amd as fa
    rnd = random.Random(seed)
    out = []
    while len(out) < n:
        B, H = rnd.choice([1, 2]), rnd.choice([1, 2, 4, 8, 12])
        Hkv = rnd.choice([h for h in (1, 2, 4, H) if H % h == 0])
        Nq, Nk = rnd.randint(1, 600), rnd.randint(1500, 6000)
        D = rnd.choice([64, 128])
        kind = rnd.choice(["none", "causal", "sliding_window", "prefix_lm"])
        window = rnd.randint(200, 4000) if kind == "sliding_window" else 0
        prefix = rnd.randint(0, 3000) if kind == "prefix_lm" else 0
        cap = rnd.choice([0.0, 0.0, 20.0, 50.0])
        slope = rnd.choice([0.0, 0.0, -0.005, 0.003])
        q = torch.empty(B, Nq, H, D, device=device(), dtype=torch.bfloat16)
        k = torch.empty(B, Nk, Hkv, D, device=device(), dtype=torch.bfloat16)
        if fa.fwd_workspace_size(q, k, k, mask=fa.Mask(kind, window=window, prefix=prefix)) > 0:
            out.append((B, Nq, Nk, H, Hkv, D, kind, window, prefix, cap, slope))
    return out


@pytest.mark.parametrize("case", range(16))
def test_fwd_bf16_key_split_fuzz(case):
    import block_sparse_attention_fmha_amd as fa
    B, Nq, Nk, H, Hkv, D, kind, W, P, cap, slope = _key_split_fuzz_cases()[case]
    seed = synth.case_seed(9, 500 + case)
    q, k, v = synth.normal_tensors(seed, [(B, Nq, H, D), (B, Nk, Hkv, D), (B, Nk, Hkv, D)], "bf16")
    om, gm = mask_pair(kind, B, Nq, Nk, W, P)
    heads = None if H <= 2 else [0, H - 1]
    o_ref, l_ref = oracle.forward(q.values, k.values, v.values, softcap=cap, bias_slope=slope, mask=om, heads=heads)
    hsel = slice(None) if heads is None else np.asarray(heads)
    announce(f"fwd bf16 key-split fuzz {case}: B={B} Nq={Nq} Nk={Nk} H={H} Hkv={Hkv} D={D} mask={kind} "
             f"window={W} prefix={P} softcap={cap} bias={slope}")
    out, lse = fa.fmha_fwd(to_dev(q), to_dev(k), to_dev(v), mask=gm, softcap=cap, bias_slope=slope)
    import torch
    torch.cuda.synchronize()
    check_bf16("O", host(out)[:, :, hsel], o_ref[:, :, hsel])
    check_bf16("LSE", host(lse)[:, hsel], l_ref[:, hsel])
