"""The C ABI without a GPU: libfmha.so loads, exports every function include/fmha.h
declares, the ctypes mirror matches the header's struct layout, and host-side argument
validation rejects bad requests before anything is launched."""
import ctypes
import os
import re

import pytest

import block_sparse_attention_fmha_amd as fa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fmha.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(fa.lib_path()):
        from block_sparse_attention_fmha_amd import build
        build.build()
    return fa.load_library()


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*([a-z_][a-z0-9_]*)\s*\(", text, flags=re.M)
    return sorted(set(names))


def test_header_declares_the_entry_points():
    assert header_functions() == sorted(fa.ENTRY_POINTS)


def test_every_declared_symbol_is_exported(lib):
    for name in header_functions():
        assert hasattr(lib, name), name


def test_abi_version_and_status_strings(lib):
    assert lib.fmha_abi_version() == fa.ABI_VERSION == 4
    assert fa.status_string(0) == "FMHA_OK"
    assert fa.status_string(-4) == "FMHA_ERR_WORKSPACE"
    assert fa.status_string(12345) == "FMHA_ERR_UNKNOWN"


def test_struct_layout_matches_header():
    # offsets the header implies for LP64 (int32 fields, 8-byte pointers / int64)
    assert ctypes.sizeof(fa.CMask) == 32
    assert ctypes.sizeof(fa.CBlockSparse) == 24 + 8 * 8
    assert fa.CFwdArgs.q.offset == 32 and fa.CFwdArgs.q_stride.offset == 72
    assert fa.CFwdArgs.scale.offset == 168 and fa.CFwdArgs.mask.offset == 184
    assert fa.CFwdArgs.block_sparse.offset == 216 and ctypes.sizeof(fa.CFwdArgs) == 224
    assert ctypes.sizeof(fa.CBwdArgs) == 32 + 96 + 24


def _args(**kw):
    a = fa.CFwdArgs()
    a.B, a.H, a.Nq, a.Nk, a.Dqk, a.Dv, a.dtype = 1, 2, 64, 64, 128, 128, fa.FMHA_BF16
    fake = 0x100000  # never dereferenced: validation fails first
    a.q = a.k = a.v = a.o = a.lse = fake
    for s in (a.q_stride, a.k_stride, a.v_stride, a.o_stride):
        s[0], s[1], s[2] = 64 * 2 * 128, 2 * 128, 128
    a.scale = 0.125
    for key, val in kw.items():
        setattr(a, key, val)
    return a


@pytest.mark.parametrize("kw,status", [
    ({"Dqk": 96, "Dv": 96}, fa.FMHA_ERR_UNSUPPORTED),
    ({"Dqk": 128, "Dv": 64}, fa.FMHA_ERR_UNSUPPORTED),
    ({"lse": None}, fa.FMHA_ERR_INVALID_ARG),
    ({"q": 0x100008}, fa.FMHA_ERR_INVALID_ARG),          # not 16-byte aligned
    ({"scale": 0.0}, fa.FMHA_ERR_INVALID_ARG),
    ({"scale": float("nan")}, fa.FMHA_ERR_INVALID_ARG),
    ({"softcap": -1.0}, fa.FMHA_ERR_INVALID_ARG),
    ({"dtype": 7}, fa.FMHA_ERR_INVALID_ARG),
    ({"kv_heads": -1}, fa.FMHA_ERR_INVALID_ARG),
    ({"kv_heads": 3}, fa.FMHA_ERR_INVALID_ARG),           # does not divide H = 2
    ({"reserved2": 1}, fa.FMHA_ERR_INVALID_ARG),
    ({"Nq": -1}, fa.FMHA_ERR_INVALID_ARG),
    ({"dtype": fa.FMHA_FP32, "Dqk": 1024, "Dv": 1024, "softcap": 30.0}, fa.FMHA_ERR_UNSUPPORTED),
])
def test_fwd_rejects_bad_arguments(lib, kw, status):
    a = _args(**kw)
    assert lib.fmha_fwd(ctypes.byref(a), None) == status


def test_fwd_rejects_misaligned_stride_and_bad_mask(lib):
    a = _args()
    a.k_stride[1] = 129  # 258-byte rows
    assert lib.fmha_fwd(ctypes.byref(a), None) == fa.FMHA_ERR_INVALID_ARG
    a = _args()
    a.mask.kind = 9
    assert lib.fmha_fwd(ctypes.byref(a), None) == fa.FMHA_ERR_INVALID_ARG
    a = _args()
    a.mask.kind = fa.MASK_KINDS["block_diagonal"]   # doc ids missing
    assert lib.fmha_fwd(ctypes.byref(a), None) == fa.FMHA_ERR_INVALID_ARG
    a = _args()
    a.mask.kind, a.mask.window = fa.MASK_KINDS["sliding_window"], -3
    assert lib.fmha_fwd(ctypes.byref(a), None) == fa.FMHA_ERR_INVALID_ARG


def test_null_and_empty_requests(lib):
    assert lib.fmha_fwd(None, None) == fa.FMHA_ERR_INVALID_ARG
    a = _args(Nq=0)
    assert lib.fmha_fwd(ctypes.byref(a), None) == fa.FMHA_OK      # nothing to compute, no launch
    a = _args(B=0)
    assert lib.fmha_fwd(ctypes.byref(a), None) == fa.FMHA_OK


def test_block_sparse_tile_constraints(lib):
    bs = fa.CBlockSparse()
    bs.tile_m, bs.tile_n, bs.n_q_tiles, bs.n_kv_tiles, bs.heads = 64, 64, 1, 1, 1
    for name in ("partial_cnt", "partial_idx", "full_cnt", "full_idx"):
        setattr(bs, name, 0x100000)
    a = _args()
    a.block_sparse = ctypes.pointer(bs)
    assert lib.fmha_fwd(ctypes.byref(a), None) == fa.FMHA_ERR_UNSUPPORTED   # tile_m not a multiple of 128
    bs.tile_m, bs.n_q_tiles = 128, 1
    bs.n_kv_tiles = 5                                                       # inconsistent with Nk / tile_n
    assert lib.fmha_fwd(ctypes.byref(a), None) == fa.FMHA_ERR_INVALID_ARG


def _align256(x):
    return (x + 255) // 256 * 256


MASK_CAUSAL, MASK_WINDOW, MASK_PREFIX = (fa.MASK_KINDS[k] for k in ("causal", "sliding_window", "prefix_lm"))


def _key_tiles(kind, window, prefix, q0, Nq, Nk, rows=256, tile=64):
    """Key tiles a 256-row query tile of the bf16 forward walks under a band mask."""
    delta = Nk - Nq
    lo, hi = 0, Nk
    if kind in (MASK_CAUSAL, MASK_WINDOW):
        hi = min(Nk, q0 + rows + delta)
    if kind == MASK_PREFIX:
        hi = min(Nk, max(prefix, q0 + rows + delta))
    if kind == MASK_WINDOW:
        lo = max(0, q0 + delta - window)
    hi = max(hi, 0)
    return max(0, -(-hi // tile) - lo // tile)


def _key_split(B, H, Nq, Nk, kind=0, window=0, prefix=0, Dv=128):
    """(parts, tiles) of the forward's key split: for grids short of the 256 CUs, the part
    count whose parts fit the CUs in one round with the largest predicted saving (tiles of
    1.5 us at Dv 128, 1.0 us at Dv 64; a split costs 5 us + 0.9 us per MiB of fp32 partial O)."""
    n_tiles = -(-Nq // 256)
    heads = B * H
    if heads * n_tiles >= 256:
        return 1, 0
    counts = [_key_tiles(kind, window, prefix, 256 * t, Nq, Nk) for t in range(n_tiles)]
    longest = max(counts)
    tile_us = 1.5 if Dv == 128 else 1.0
    best, best_saving = (1, 0), 0.0
    for s in range(2, 17):
        tiles = -(-longest // s)
        if tiles < 4:
            break
        ns = [min(16, max(1, -(-c // tiles))) for c in counts]
        if sum(ns) * heads > 256:
            continue
        piece = max(-(-c // n) for c, n in zip(counts, ns))
        part_rows = sum(n * 256 for n in ns if n > 1)
        part_mib = float(part_rows * heads) * Dv * 4 / (1 << 20)
        saving = (longest - piece) * tile_us - (5.0 + 0.9 * part_mib)
        if saving > best_saving:
            best, best_saving = (-(-longest // tiles), tiles), saving
    return best


@pytest.mark.parametrize("kw,splits", [
    ({"H": 16, "Nq": 1024, "Nk": 8192}, 4),      # 64 tiles of 128 key tiles: 4 parts of 32 fill 256 CUs
    ({"H": 16, "Nq": 256, "Nk": 32768}, 16),     # short query side, long keys: capped at 16
    ({"H": 2, "Nq": 129, "Nk": 8000}, 16),       # 2 tiles of 125 key tiles: parts of 8
    ({"H": 16, "Nq": 1024, "Nk": 1024}, 1),      # 16 key tiles: the partials cost more than they save
    ({"H": 16, "Nq": 1024, "Nk": 1024, "mask": MASK_CAUSAL}, 1),
    ({"H": 16, "Nq": 2048, "Nk": 2048}, 1),
    ({"H": 16, "Nq": 2048, "Nk": 2048, "mask": MASK_CAUSAL}, 2),   # the 4 longest tiles in 2 parts
    ({"H": 16, "Nq": 4096, "Nk": 4096, "mask": MASK_CAUSAL}, 1),   # 256 tiles fill the CUs
    ({"H": 2, "Nq": 4096, "Nk": 4096, "mask": MASK_CAUSAL}, 8),    # 32 tiles, longest 64
    ({"H": 16, "Nq": 4096, "Nk": 4096, "mask": MASK_WINDOW, "window": 1024}, 1),
    ({"H": 16, "Nq": 16384, "Nk": 16384, "mask": MASK_CAUSAL}, 1),
    ({"H": 16, "Nq": 1024, "Nk": 8192, "Dqk": 64, "Dv": 64}, 4),
    ({"H": 16, "Nq": 1024, "Nk": 8192, "Dqk": 192, "Dv": 128}, 1),
    ({"H": 16, "Nq": 1024, "Nk": 8192, "dtype": fa.FMHA_FP32}, 1),
    ({"H": 16, "Nq": 1024, "Nk": 8192, "lse": None}, 0),   # invalid: no workspace
])
def test_fwd_workspace_size(lib, kw, splits):
    kw = dict(kw)
    kind, window = kw.pop("mask", 0), kw.pop("window", 0)
    a = _args(**kw)
    a.mask.kind, a.mask.window = kind, window
    for s in (a.q_stride, a.k_stride, a.v_stride, a.o_stride):
        s[0], s[1] = a.Nq * a.H * 128 * 2 if s is a.q_stride else max(a.Nq, a.Nk) * a.H * 128 * 2, a.H * 128 * 2
    got = lib.fmha_fwd_workspace_size(ctypes.byref(a))
    if splits <= 1:
        assert got == 0
        return
    if a.dtype == fa.FMHA_BF16 and a.Dqk == a.Dv:
        assert _key_split(a.B, a.H, a.Nq, a.Nk, kind, window, Dv=a.Dv)[0] == splits
    rows = a.B * a.H * -(-a.Nq // 256) * splits * 256   # 256-row slots per query tile and part
    assert got == _align256(_align256(rows * a.Dv * 4) + rows * 4)


def test_fwd_key_split_planner_random_sweep(lib):
    """The library's key-split plan (seen through the workspace size) equals the host model
    above on 600 random shapes and masks: B, H, Nq, Nk, Dv, mask kind, window and prefix."""
    import random
    rnd = random.Random(20261203)
    kinds = [0, MASK_CAUSAL, MASK_WINDOW, MASK_PREFIX, fa.MASK_KINDS["block_diagonal"]]
    split_seen = 0
    for _ in range(600):
        B, H = rnd.choice([1, 1, 2, 4]), rnd.choice([1, 2, 3, 8, 16, 32])
        Nq = rnd.choice([1, 7, 64, 129, 256, 300, 512, 1000, 1024, 2048, 4096])
        Nk = rnd.choice([1, 63, 64, 500, 1024, 2048, 4097, 8192, 16384, 65536])
        D = rnd.choice([64, 128])
        kind = rnd.choice(kinds)
        window = rnd.choice([0, 100, 1024, 3000]) if kind == MASK_WINDOW else 0
        prefix = rnd.choice([0, 200, 5000]) if kind == MASK_PREFIX else 0
        a = _args(B=B, H=H, Nq=Nq, Nk=Nk, Dqk=D, Dv=D)
        a.mask.kind, a.mask.window, a.mask.prefix = kind, window, prefix
        if kind == fa.MASK_KINDS["block_diagonal"]:
            a.mask.doc_q = a.mask.doc_k = 0x100000   # never dereferenced by the size query
        for st, rows in ((a.q_stride, Nq), (a.o_stride, Nq), (a.k_stride, Nk), (a.v_stride, Nk)):
            st[0], st[1], st[2] = rows * H * D, H * D, D
        got = lib.fmha_fwd_workspace_size(ctypes.byref(a))
        parts, _ = _key_split(B, H, Nq, Nk, kind, window, prefix, Dv=D)
        if parts <= 1:
            assert got == 0, (B, H, Nq, Nk, D, kind, window, prefix)
        else:
            split_seen += 1
            rows_ = B * H * -(-Nq // 256) * parts * 256
            assert got == _align256(_align256(rows_ * D * 4) + rows_ * 4), (B, H, Nq, Nk, D, kind, window, prefix)
    assert split_seen > 50   # the sweep exercises the split path, not only the unsplit one


def test_fwd_rejects_sequence_stride_beyond_32bit_tile_offsets(lib):
    a = _args()
    a.k_stride[1] = (1 << 31) // (2 * 64)          # 64 rows of bf16 reach 2^31 bytes
    a.k_stride[0] = a.k_stride[1] * 64
    assert lib.fmha_fwd(ctypes.byref(a), None) == fa.FMHA_ERR_UNSUPPORTED
    # (requests that pass validation are not made here: with fake pointers they would
    # launch on a machine that has a GPU)


def test_block_sparse_list_granularity(lib):
    # forward lists need tile_m % 128 and tile_n % 64 (accepted shapes such as 384 x 192
    # are exercised by the GPU tests)
    bs = fa.CBlockSparse()
    for name in ("partial_cnt", "partial_idx", "full_cnt", "full_idx"):
        setattr(bs, name, 0x100000)
    a = _args()
    a.block_sparse = ctypes.pointer(bs)
    for tm, tn in ((128, 32), (192, 64), (64, 128)):
        bs.tile_m, bs.tile_n, bs.heads = tm, tn, 1
        bs.n_q_tiles, bs.n_kv_tiles = -(-a.Nq // tm), -(-a.Nk // tn)
        assert lib.fmha_fwd(ctypes.byref(a), None) == fa.FMHA_ERR_UNSUPPORTED, (tm, tn)


def test_bwd_and_splitkv_workspace_checks(lib):
    a = _args()
    g = fa.CBwdArgs()
    g.dout = g.dq = g.dk = g.dv = 0x100000
    for s in (g.do_stride, g.dq_stride, g.dk_stride, g.dv_stride):
        s[0], s[1], s[2] = 64 * 2 * 128, 2 * 128, 128
    need = lib.fmha_bwd_workspace_size(1, 2, 64)
    assert need >= 1 * 2 * 64 * 4 and need % 256 == 0
    g.workspace, g.workspace_bytes = 0x200000, need - 1
    assert lib.fmha_bwd(ctypes.byref(a), ctypes.byref(g), None) == fa.FMHA_ERR_WORKSPACE
    g.workspace, g.workspace_bytes = 0x200008, need   # large enough but not 16-byte aligned
    assert lib.fmha_bwd(ctypes.byref(a), ctypes.byref(g), None) == fa.FMHA_ERR_WORKSPACE
    assert lib.fmha_bwd(ctypes.byref(a), None, None) == fa.FMHA_ERR_INVALID_ARG
    need = lib.fmha_fwd_splitkv_workspace_size(1, 2, 64, 128, 4)
    assert need >= 1 * 2 * 4 * 64 * (128 + 1) * 4
    assert lib.fmha_fwd_splitkv(ctypes.byref(a), 4, ctypes.c_void_p(0x200000), need - 1, None) == fa.FMHA_ERR_WORKSPACE
    assert lib.fmha_fwd_splitkv(ctypes.byref(a), 0, ctypes.c_void_p(0x200000), need, None) == fa.FMHA_ERR_INVALID_ARG
    assert lib.fmha_fwd_splitkv(ctypes.byref(a), 65, ctypes.c_void_p(0x200000), need, None) == fa.FMHA_ERR_INVALID_ARG


def test_build_block_mask_argument_checks(lib):
    m = fa.CMask()
    out = fa.CBlockSparse()
    assert lib.build_block_mask(ctypes.byref(m), 1, 1, 128, 128, 64, 64, ctypes.byref(out), None) == fa.FMHA_ERR_INVALID_ARG
    assert lib.build_block_mask(None, 1, 1, 128, 128, 64, 64, ctypes.byref(out), None) == fa.FMHA_ERR_INVALID_ARG
    for name in ("partial_cnt", "partial_idx", "full_cnt", "full_idx", "t_partial_cnt", "t_partial_idx",
                 "t_full_cnt", "t_full_idx"):
        setattr(out, name, 0x100000)
    assert lib.build_block_mask(ctypes.byref(m), 1, 1, 128, 128, 0, 64, ctypes.byref(out), None) == fa.FMHA_ERR_INVALID_ARG


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(fa, "LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(fa, "_LIB", None)
    with pytest.raises(RuntimeError, match="missing"):
        fa.load_library()


def test_ctypes_layout_matches_c_compiler(tmp_path):
    import shutil
    import subprocess
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no host C compiler")
    src = tmp_path / "layout.c"
    src.write_text('#include <stddef.h>\n#include <stdio.h>\n#include "fmha.h"\n'
                   "#define P(s, f) printf(#s \".\" #f \" %zu\\n\", offsetof(s, f))\n"
                   "int main(void) {\n"
                   "  P(fmha_fwd_args, kv_heads); P(fmha_fwd_args, q); P(fmha_fwd_args, lse); P(fmha_fwd_args, q_stride);"
                   "  P(fmha_fwd_args, o_stride); P(fmha_fwd_args, scale); P(fmha_fwd_args, mask);"
                   "  P(fmha_fwd_args, block_sparse); P(fmha_bwd_args, workspace);"
                   "  P(fmha_bwd_args, workspace_bytes); P(fmha_block_sparse, partial_cnt);"
                   "  P(fmha_block_sparse, t_full_idx); P(fmha_mask, doc_k);\n"
                   '  printf("sizeof.fwd %zu\\nsizeof.bwd %zu\\nsizeof.bs %zu\\nsizeof.mask %zu\\n",'
                   " sizeof(fmha_fwd_args), sizeof(fmha_bwd_args), sizeof(fmha_block_sparse), sizeof(fmha_mask));\n"
                   "  return 0; }\n")
    exe = tmp_path / "layout"
    subprocess.run([cc, "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)], check=True)
    got = dict(line.split() for line in subprocess.run([str(exe)], capture_output=True, text=True,
                                                       check=True).stdout.splitlines())
    want = {
        "fmha_fwd_args.kv_heads": fa.CFwdArgs.kv_heads.offset,
        "fmha_fwd_args.q": fa.CFwdArgs.q.offset, "fmha_fwd_args.lse": fa.CFwdArgs.lse.offset,
        "fmha_fwd_args.q_stride": fa.CFwdArgs.q_stride.offset,
        "fmha_fwd_args.o_stride": fa.CFwdArgs.o_stride.offset,
        "fmha_fwd_args.scale": fa.CFwdArgs.scale.offset, "fmha_fwd_args.mask": fa.CFwdArgs.mask.offset,
        "fmha_fwd_args.block_sparse": fa.CFwdArgs.block_sparse.offset,
        "fmha_bwd_args.workspace": fa.CBwdArgs.workspace.offset,
        "fmha_bwd_args.workspace_bytes": fa.CBwdArgs.workspace_bytes.offset,
        "fmha_block_sparse.partial_cnt": fa.CBlockSparse.partial_cnt.offset,
        "fmha_block_sparse.t_full_idx": fa.CBlockSparse.t_full_idx.offset,
        "fmha_mask.doc_k": fa.CMask.doc_k.offset,
        "sizeof.fwd": ctypes.sizeof(fa.CFwdArgs), "sizeof.bwd": ctypes.sizeof(fa.CBwdArgs),
        "sizeof.bs": ctypes.sizeof(fa.CBlockSparse), "sizeof.mask": ctypes.sizeof(fa.CMask),
    }
    assert {k: int(v) for k, v in got.items()} == want


def test_varlen_argument_checks(lib):
    a = _args()
    vl = fa.CVarlen()
    vl.cu_seqlens_q = vl.cu_seqlens_k = 0x200000
    vl.total_q, vl.reserved = 64, 0
    assert lib.fmha_fwd_varlen(ctypes.byref(a), None, None) == fa.FMHA_ERR_INVALID_ARG
    bad = fa.CVarlen()
    bad.cu_seqlens_q, bad.cu_seqlens_k, bad.total_q = 0x200000, None, 64
    assert lib.fmha_fwd_varlen(ctypes.byref(a), ctypes.byref(bad), None) == fa.FMHA_ERR_INVALID_ARG
    bad.cu_seqlens_k, bad.total_q = 0x200000, -1
    assert lib.fmha_fwd_varlen(ctypes.byref(a), ctypes.byref(bad), None) == fa.FMHA_ERR_INVALID_ARG
    bad.total_q, bad.reserved = 64, 1
    assert lib.fmha_fwd_varlen(ctypes.byref(a), ctypes.byref(bad), None) == fa.FMHA_ERR_INVALID_ARG
    for kw in ({"dtype": fa.FMHA_FP32},):
        b = _args(**kw)
        assert lib.fmha_fwd_varlen(ctypes.byref(b), ctypes.byref(vl), None) == fa.FMHA_ERR_UNSUPPORTED
    b = _args()
    b.mask.kind = fa.MASK_KINDS["block_diagonal"]
    b.mask.doc_q = b.mask.doc_k = 0x200000
    assert lib.fmha_fwd_varlen(ctypes.byref(b), ctypes.byref(vl), None) == fa.FMHA_ERR_UNSUPPORTED


def test_varlen_struct_layout(tmp_path):
    import shutil
    import subprocess
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no host C compiler")
    src = tmp_path / "vl.c"
    src.write_text('#include <stddef.h>\n#include <stdio.h>\n#include "fmha.h"\n'
                   'int main(void) { printf("%zu %zu %zu %zu %zu\\n", offsetof(fmha_varlen, total_q),'
                   ' offsetof(fmha_varlen, reserved), offsetof(fmha_varlen, seqused_q),'
                   ' offsetof(fmha_varlen, seqused_k), sizeof(fmha_varlen)); return 0; }\n')
    exe = tmp_path / "vl"
    subprocess.run([cc, "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)], check=True)
    got = [int(x) for x in subprocess.run([str(exe)], capture_output=True, text=True, check=True).stdout.split()]
    assert got == [fa.CVarlen.total_q.offset, fa.CVarlen.reserved.offset, fa.CVarlen.seqused_q.offset,
                   fa.CVarlen.seqused_k.offset, ctypes.sizeof(fa.CVarlen)]


def test_backward_rejects_grouped_heads_with_per_head_lists(lib):
    # grouped K/V heads walk a whole group in one dK/dV workgroup: head-broadcast lists only
    a = _args(kv_heads=1)
    bs = fa.CBlockSparse()
    bs.tile_m, bs.tile_n, bs.n_q_tiles, bs.n_kv_tiles, bs.heads = 128, 128, 1, 1, 2
    a.block_sparse = ctypes.pointer(bs)
    g = fa.CBwdArgs()
    assert lib.fmha_bwd(ctypes.byref(a), ctypes.byref(g), None) == fa.FMHA_ERR_UNSUPPORTED


def test_backward_one_empty_side_checks_only_that_sides_buffers(lib):
    # Nk = 0: dQ (written as 0) and dO must be given, K / V / dK / dV may be NULL;
    # Nq = 0: dK / dV (written as 0) must be given. Both rejections precede any device use.
    fake = 0x100000
    a = _args(Nk=0, k=None, v=None)
    g = fa.CBwdArgs()
    g.dout = fake
    assert lib.fmha_bwd(ctypes.byref(a), ctypes.byref(g), None) == fa.FMHA_ERR_INVALID_ARG   # no dQ
    a = _args(Nq=0, q=None, o=None, lse=None)
    g = fa.CBwdArgs()
    g.dk = fake
    assert lib.fmha_bwd(ctypes.byref(a), ctypes.byref(g), None) == fa.FMHA_ERR_INVALID_ARG   # no dV
    a = _args(Nq=0, Nk=0)
    assert lib.fmha_bwd(ctypes.byref(a), ctypes.byref(fa.CBwdArgs()), None) == fa.FMHA_OK   # nothing to write


@pytest.mark.parametrize("bad", ["neg_stride", "odd_stride", "misaligned_k", "null_v"])
def test_backward_without_queries_still_validates_keys(lib, bad):
    # Nq = 0, Nk > 0: the dK / dV pass still reads K and V (and writes zeros), so their
    # pointers and strides are checked before anything is launched
    fake = 0x100000
    a = _args(Nq=0, q=None, o=None, lse=None)
    if bad == "neg_stride":
        a.k_stride[1] = -2 * 128
    elif bad == "odd_stride":
        a.v_stride[1] = 2 * 128 + 2
    elif bad == "misaligned_k":
        a.k = fake + 8
    else:
        a.v = None
    g = fa.CBwdArgs()
    g.dk = g.dv = fake
    for s in (g.do_stride, g.dq_stride, g.dk_stride, g.dv_stride):
        s[0], s[1], s[2] = 64 * 2 * 128, 2 * 128, 128
    g.workspace, g.workspace_bytes = 0x200000, lib.fmha_bwd_workspace_size(1, 2, 0)
    assert lib.fmha_bwd(ctypes.byref(a), ctypes.byref(g), None) == fa.FMHA_ERR_INVALID_ARG


def test_noalloc_splitkv_rejects_requests_beyond_its_scratch(lib):
    # the size check needs no device: partials of B*H*Nq*splits rows of (Dv + 1) fp32
    cap = lib.fmha_fwd_splitkv_noalloc_max_bytes()
    assert cap == 16 << 20
    a = _args(B=64, H=64, Nq=1, Nk=4096)
    need = lib.fmha_fwd_splitkv_workspace_size(64, 64, 1, 128, 16)
    assert need > cap
    assert lib.fmha_fwd_splitkv_noalloc(ctypes.byref(a), 16, None) == fa.FMHA_ERR_SCRATCH_TOO_SMALL
    assert fa.status_string(fa.FMHA_ERR_SCRATCH_TOO_SMALL) == "FMHA_ERR_SCRATCH_TOO_SMALL"
    assert lib.fmha_fwd_splitkv_noalloc(ctypes.byref(a), 0, None) == fa.FMHA_ERR_INVALID_ARG
