"""Python binding of libfmha.so: fused masked attention for AMD MI355X (gfx950).

Argument marshalling only: every step of the computation runs in the HIP kernels
behind the C ABI declared in ``include/fmha.h``. PyTorch provides device memory and
the current HIP stream. Each function has the name of the C entry point it calls:

    fmha_fwd(q, k, v, ...)                   -> (out, lse)
    fmha_bwd(q, k, v, out, lse, dout, ...)   -> (dq, dk, dv)
    fmha_fwd_splitkv(q, k, v, num_splits...) -> (out, lse)
    build_block_mask(mask, B, Nq, Nk, ...)   -> BlockSparse

Tensors are ``[batch, seq, head, dim]`` with a contiguous head dim (any batch / seq /
head strides whose byte size is a multiple of 16). If libfmha.so is missing the calls
raise: there is no fallback path.
"""
from __future__ import annotations

import ctypes
import math
import os
from dataclasses import dataclass, field

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libfmha.so")

FMHA_OK, FMHA_ERR_INVALID_ARG, FMHA_ERR_UNSUPPORTED, FMHA_ERR_HIP, FMHA_ERR_WORKSPACE = 0, -1, -2, -3, -4
FMHA_ERR_SCRATCH_TOO_SMALL = -5
FMHA_BF16, FMHA_FP32 = 0, 1
MASK_KINDS = {"none": 0, "causal": 1, "sliding_window": 2, "block_diagonal": 3, "prefix_lm": 4}
ABI_VERSION = 4   # the struct layouts and entry points below (fmha_abi_version of include/fmha.h)
ENTRY_POINTS = ("fmha_fwd", "fmha_fwd_workspace_size", "fmha_fwd_with_workspace", "fmha_bwd",
                "fmha_bwd_workspace_size", "fmha_fwd_splitkv",
                "fmha_fwd_splitkv_workspace_size", "fmha_fwd_splitkv_noalloc", "fmha_fwd_splitkv_noalloc_max_bytes",
                "fmha_fwd_varlen", "fmha_bwd_varlen", "build_block_mask", "fmha_status_string", "fmha_abi_version")


class FmhaError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what} failed: {status_string(status)} ({status})")
        self.status = status


# ------------------------------------------------------------------ C structs (fmha.h)

class CMask(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int32), ("window", ctypes.c_int32), ("prefix", ctypes.c_int32),
                ("reserved", ctypes.c_int32), ("doc_q", ctypes.c_void_p), ("doc_k", ctypes.c_void_p)]


class CBlockSparse(ctypes.Structure):
    _fields_ = [("tile_m", ctypes.c_int32), ("tile_n", ctypes.c_int32),
                ("n_q_tiles", ctypes.c_int32), ("n_kv_tiles", ctypes.c_int32),
                ("heads", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("partial_cnt", ctypes.c_void_p), ("partial_idx", ctypes.c_void_p),
                ("full_cnt", ctypes.c_void_p), ("full_idx", ctypes.c_void_p),
                ("t_partial_cnt", ctypes.c_void_p), ("t_partial_idx", ctypes.c_void_p),
                ("t_full_cnt", ctypes.c_void_p), ("t_full_idx", ctypes.c_void_p)]


Strides3 = ctypes.c_int64 * 3


class CFwdArgs(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("H", ctypes.c_int32), ("Nq", ctypes.c_int32),
                ("Nk", ctypes.c_int32), ("Dqk", ctypes.c_int32), ("Dv", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("kv_heads", ctypes.c_int32),
                ("q", ctypes.c_void_p), ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
                ("o", ctypes.c_void_p), ("lse", ctypes.c_void_p),
                ("q_stride", Strides3), ("k_stride", Strides3), ("v_stride", Strides3),
                ("o_stride", Strides3),
                ("scale", ctypes.c_float), ("softcap", ctypes.c_float), ("bias_slope", ctypes.c_float),
                ("reserved2", ctypes.c_int32), ("mask", CMask),
                ("block_sparse", ctypes.POINTER(CBlockSparse))]


class CVarlen(ctypes.Structure):
    _fields_ = [("cu_seqlens_q", ctypes.c_void_p), ("cu_seqlens_k", ctypes.c_void_p),
                ("total_q", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("seqused_q", ctypes.c_void_p), ("seqused_k", ctypes.c_void_p)]


class CBwdArgs(ctypes.Structure):
    _fields_ = [("dout", ctypes.c_void_p), ("dq", ctypes.c_void_p), ("dk", ctypes.c_void_p),
                ("dv", ctypes.c_void_p), ("do_stride", Strides3), ("dq_stride", Strides3),
                ("dk_stride", Strides3), ("dv_stride", Strides3),
                ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_size_t),
                ("stage_events", ctypes.c_void_p)]


# ------------------------------------------------------------------ library loading

_LIB = None


def lib_path() -> str:
    return LIB_PATH


def load_library():
    """Load libfmha.so (raises if it has not been built)."""
    global _LIB
    if _LIB is not None:
        return _LIB
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                           "`python -m block_sparse_attention_fmha_amd.build` (no fallback path exists)")
    # torch first: its HIP runtime is then the one the library's HIP calls resolve to (loading
    # the library alone first would bring in a second runtime copy that sees no device once
    # torch has set up its own)
    import torch  # noqa: F401
    lib = ctypes.CDLL(LIB_PATH)
    lib.fmha_fwd.argtypes = [ctypes.POINTER(CFwdArgs), ctypes.c_void_p]
    lib.fmha_fwd.restype = ctypes.c_int
    lib.fmha_fwd_workspace_size.argtypes = [ctypes.POINTER(CFwdArgs)]
    lib.fmha_fwd_workspace_size.restype = ctypes.c_size_t
    lib.fmha_fwd_with_workspace.argtypes = [ctypes.POINTER(CFwdArgs), ctypes.c_void_p, ctypes.c_size_t,
                                            ctypes.c_void_p]
    lib.fmha_fwd_with_workspace.restype = ctypes.c_int
    lib.fmha_bwd.argtypes = [ctypes.POINTER(CFwdArgs), ctypes.POINTER(CBwdArgs), ctypes.c_void_p]
    lib.fmha_bwd.restype = ctypes.c_int
    lib.fmha_bwd_workspace_size.argtypes = [ctypes.c_int32] * 3
    lib.fmha_bwd_workspace_size.restype = ctypes.c_size_t
    lib.fmha_fwd_splitkv.argtypes = [ctypes.POINTER(CFwdArgs), ctypes.c_int32, ctypes.c_void_p,
                                     ctypes.c_size_t, ctypes.c_void_p]
    lib.fmha_fwd_splitkv.restype = ctypes.c_int
    lib.fmha_fwd_varlen.argtypes = [ctypes.POINTER(CFwdArgs), ctypes.POINTER(CVarlen), ctypes.c_void_p]
    lib.fmha_fwd_varlen.restype = ctypes.c_int
    lib.fmha_bwd_varlen.argtypes = [ctypes.POINTER(CFwdArgs), ctypes.POINTER(CBwdArgs), ctypes.POINTER(CVarlen),
                                    ctypes.c_void_p]
    lib.fmha_bwd_varlen.restype = ctypes.c_int
    lib.fmha_fwd_splitkv_noalloc.argtypes = [ctypes.POINTER(CFwdArgs), ctypes.c_int32, ctypes.c_void_p]
    lib.fmha_fwd_splitkv_noalloc.restype = ctypes.c_int
    lib.fmha_fwd_splitkv_noalloc_max_bytes.argtypes = []
    lib.fmha_fwd_splitkv_noalloc_max_bytes.restype = ctypes.c_size_t
    lib.fmha_fwd_splitkv_workspace_size.argtypes = [ctypes.c_int32] * 5
    lib.fmha_fwd_splitkv_workspace_size.restype = ctypes.c_size_t
    lib.build_block_mask.argtypes = [ctypes.POINTER(CMask)] + [ctypes.c_int32] * 6 + [
        ctypes.POINTER(CBlockSparse), ctypes.c_void_p]
    lib.build_block_mask.restype = ctypes.c_int
    lib.fmha_status_string.argtypes = [ctypes.c_int]
    lib.fmha_status_string.restype = ctypes.c_char_p
    lib.fmha_abi_version.argtypes = []
    lib.fmha_abi_version.restype = ctypes.c_int
    if lib.fmha_abi_version() != ABI_VERSION:
        raise RuntimeError(f"{LIB_PATH} has ABI version {lib.fmha_abi_version()}, this binding expects "
                           f"{ABI_VERSION}: rebuild it with `python -m block_sparse_attention_fmha_amd.build`")
    _LIB = lib
    return lib


def status_string(status: int) -> str:
    return load_library().fmha_status_string(status).decode()


def _check(status: int, what: str):
    if status != FMHA_OK:
        raise FmhaError(status, what)


# ------------------------------------------------------------------ argument helpers

@dataclass
class Mask:
    """Element mask: kind in MASK_KINDS; window W; prefix P; document ids ([B,Nq], [B,Nk]
    int32 device tensors) for block_diagonal."""
    kind: str = "none"
    window: int = 0
    prefix: int = 0
    doc_q: object = field(default=None, repr=False)
    doc_k: object = field(default=None, repr=False)

    def to_c(self) -> CMask:
        if self.kind not in MASK_KINDS:
            raise ValueError(f"unknown mask kind {self.kind!r}")
        m = CMask()
        m.kind = MASK_KINDS[self.kind]
        m.window = int(self.window)
        m.prefix = int(self.prefix)
        m.reserved = 0
        if self.kind == "block_diagonal":
            dq = self.doc_q
            dk = self.doc_k if self.doc_k is not None else dq
            for t in (dq, dk):
                _need_device(t, "doc ids")
                if str(t.dtype) != "torch.int32" or not t.is_contiguous():
                    raise ValueError("doc ids must be contiguous int32 device tensors")
            m.doc_q, m.doc_k = dq.data_ptr(), dk.data_ptr()
        return m


def _need_device(t, what):
    if t is None or not getattr(t, "is_cuda", False):
        raise ValueError(f"{what} must be a device tensor")


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return FMHA_BF16
    if t.dtype == torch.float32:
        return FMHA_FP32
    raise ValueError(f"unsupported dtype {t.dtype}")


def _strides(t) -> Strides3:
    if t.dim() != 4 or t.stride(3) != 1:
        raise ValueError("expected a [batch, seq, head, dim] tensor with a contiguous head dim")
    return Strides3(t.stride(0), t.stride(1), t.stride(2))


def _stream(stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


@dataclass
class BlockSparse:
    """Block-sparse tile lists on the device (int32), forward and transposed."""
    tile_m: int
    tile_n: int
    n_q_tiles: int
    n_kv_tiles: int
    heads: int
    partial_cnt: object
    partial_idx: object
    full_cnt: object
    full_idx: object
    t_partial_cnt: object
    t_partial_idx: object
    t_full_cnt: object
    t_full_idx: object

    def to_c(self) -> CBlockSparse:
        c = CBlockSparse()
        c.tile_m, c.tile_n = self.tile_m, self.tile_n
        c.n_q_tiles, c.n_kv_tiles, c.heads, c.reserved = self.n_q_tiles, self.n_kv_tiles, self.heads, 0
        for name in ("partial_cnt", "partial_idx", "full_cnt", "full_idx", "t_partial_cnt",
                     "t_partial_idx", "t_full_cnt", "t_full_idx"):
            t = getattr(self, name)
            setattr(c, name, t.data_ptr() if t is not None else None)
        return c


def _fwd_args(q, k, v, out, lse, scale, softcap, bias_slope, mask, block_sparse):
    """Argument block of a forward call. out / lse None (size queries only): q's address and
    the contiguous [B, Nq, H, Dv] strides stand in for them; nothing is read or written."""
    size_query = out is None
    for t, n in ((q, "q"), (k, "k"), (v, "v")) + (() if size_query else ((out, "out"), (lse, "lse"))):
        _need_device(t, n)
    if not (q.dtype == k.dtype == v.dtype and (size_query or out.dtype == q.dtype)):
        raise ValueError("q, k, v and out must share one dtype")
    B, Nq, H, Dqk = q.shape
    Nk, Hkv, Dv = k.shape[1], k.shape[2], v.shape[3]
    if k.shape != (B, Nk, Hkv, Dqk) or v.shape != (B, Nk, Hkv, Dv) or (
            not size_query and out.shape != (B, Nq, H, Dv)):
        raise ValueError("inconsistent q / k / v / out shapes")
    if not size_query and (tuple(lse.shape) != (B, H, Nq) or str(lse.dtype) != "torch.float32"
                           or not lse.is_contiguous()):
        raise ValueError("lse must be a contiguous float32 [B, H, Nq] tensor")
    a = CFwdArgs()
    a.B, a.H, a.Nq, a.Nk, a.Dqk, a.Dv = B, H, Nq, Nk, Dqk, Dv
    a.dtype = _dtype_code(q)
    a.kv_heads = 0 if Hkv == H else Hkv   # grouped K/V heads: the library decides support
    a.reserved2 = 0
    o_ptr, lse_ptr = (q.data_ptr(), q.data_ptr()) if size_query else (out.data_ptr(), lse.data_ptr())
    a.q, a.k, a.v, a.o, a.lse = q.data_ptr(), k.data_ptr(), v.data_ptr(), o_ptr, lse_ptr
    o_stride = Strides3(Nq * H * Dv, H * Dv, Dv) if size_query else _strides(out)
    a.q_stride, a.k_stride, a.v_stride, a.o_stride = _strides(q), _strides(k), _strides(v), o_stride
    a.scale = float(1.0 / math.sqrt(Dqk) if scale is None else scale)
    a.softcap = float(softcap or 0.0)
    a.bias_slope = float(bias_slope or 0.0)
    a.mask = (mask or Mask()).to_c()
    keep = None
    if block_sparse is not None:
        keep = block_sparse.to_c()
        a.block_sparse = ctypes.pointer(keep)
    return a, keep


# ------------------------------------------------------------------ entry points

def fmha_fwd(q, k, v, *, scale=None, softcap=0.0, bias_slope=0.0, mask: Mask | None = None,
             block_sparse: BlockSparse | None = None, out=None, lse=None, stream=None,
             key_split: bool = True, workspace=None):
    """Forward: returns (out [B,Nq,H,Dv], lse [B,H,Nq] fp32).

    With ``key_split`` (the default) a grid too short for the GPU splits the key range
    (``fmha_fwd_with_workspace``); the workspace is allocated here unless ``workspace`` (a
    uint8 device tensor of at least ``fmha_fwd_workspace_size`` bytes) is given. With
    ``key_split=False`` the call is plain ``fmha_fwd``."""
    import torch
    B, Nq, H, _ = q.shape
    Dv = v.shape[3]
    if out is None:
        out = torch.empty((B, Nq, H, Dv), dtype=q.dtype, device=q.device)
    if lse is None:
        lse = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device)
    a, _keep = _fwd_args(q, k, v, out, lse, scale, softcap, bias_slope, mask, block_sparse)
    lib = load_library()
    need = lib.fmha_fwd_workspace_size(ctypes.byref(a)) if key_split else 0
    if need == 0:
        _check(lib.fmha_fwd(ctypes.byref(a), _stream(stream)), "fmha_fwd")
        return out, lse
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    _check(lib.fmha_fwd_with_workspace(ctypes.byref(a), ctypes.c_void_p(workspace.data_ptr()), need,
                                       _stream(stream)), "fmha_fwd_with_workspace")
    return out, lse


def fwd_workspace_size(q, k, v, *, mask: Mask | None = None, block_sparse: BlockSparse | None = None) -> int:
    """Bytes of workspace the key-split forward uses for these shapes (0: no split)."""
    a, _keep = _fwd_args(q, k, v, None, None, None, 0.0, 0.0, mask, block_sparse)
    return int(load_library().fmha_fwd_workspace_size(ctypes.byref(a)))


def fmha_bwd(q, k, v, out, lse, dout, *, scale=None, softcap=0.0, bias_slope=0.0,
             mask: Mask | None = None, block_sparse: BlockSparse | None = None,
             dq=None, dk=None, dv=None, workspace=None, stream=None, stage_events=None):
    """Backward from the saved LSE: returns (dq, dk, dv), bf16, shaped like q, k, v.
    ``stage_events``: optional 4 torch.cuda.Event objects recorded around the three
    backward kernels (preprocess, dK/dV, dQ) for per-kernel timing."""
    import torch
    lib = load_library()
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    B, Nq, H, _ = q.shape
    need = lib.fmha_bwd_workspace_size(B, H, Nq)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    for t, n in ((dout, "dout"), (dq, "dq"), (dk, "dk"), (dv, "dv"), (workspace, "workspace")):
        _need_device(t, n)
    if dout.shape != out.shape or dq.shape != q.shape or dk.shape != k.shape or dv.shape != v.shape:
        raise ValueError("gradient shapes must match q / k / v / out")
    a, _keep = _fwd_args(q, k, v, out, lse, scale, softcap, bias_slope, mask, block_sparse)
    g = CBwdArgs()
    g.dout, g.dq, g.dk, g.dv = dout.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr()
    g.do_stride, g.dq_stride, g.dk_stride, g.dv_stride = _strides(dout), _strides(dq), _strides(dk), _strides(dv)
    g.workspace = workspace.data_ptr()
    g.workspace_bytes = workspace.numel() * workspace.element_size()
    ev_arr = None
    if stage_events is not None:
        if len(stage_events) != 4:
            raise ValueError("stage_events needs 4 events")
        ev_arr = (ctypes.c_void_p * 4)(*[_event_handle(e) for e in stage_events])
        g.stage_events = ctypes.cast(ev_arr, ctypes.c_void_p)
    _check(lib.fmha_bwd(ctypes.byref(a), ctypes.byref(g), _stream(stream)), "fmha_bwd")
    return dq, dk, dv


def _event_handle(ev) -> int:
    """Raw hipEvent_t of a torch.cuda.Event (created on first use)."""
    if getattr(ev, "cuda_event", 0) == 0:
        import torch
        ev.record(torch.cuda.current_stream())   # materialise the handle
    return int(ev.cuda_event)


def fmha_fwd_splitkv(q, k, v, num_splits: int, *, scale=None, mask: Mask | None = None,
                     out=None, lse=None, workspace=None, stream=None):
    """Split-KV forward (partials + LSE-weighted combine): returns (out, lse)."""
    import torch
    lib = load_library()
    B, Nq, H, _ = q.shape
    Dv = v.shape[3]
    if out is None:
        out = torch.empty((B, Nq, H, Dv), dtype=q.dtype, device=q.device)
    if lse is None:
        lse = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device)
    need = lib.fmha_fwd_splitkv_workspace_size(B, H, Nq, Dv, num_splits)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    _need_device(workspace, "workspace")
    a, _keep = _fwd_args(q, k, v, out, lse, scale, 0.0, 0.0, mask, None)
    _check(lib.fmha_fwd_splitkv(ctypes.byref(a), int(num_splits), ctypes.c_void_p(workspace.data_ptr()),
                                workspace.numel() * workspace.element_size(), _stream(stream)),
           "fmha_fwd_splitkv")
    return out, lse


def fmha_fwd_splitkv_noalloc(q, k, v, num_splits: int, *, scale=None, mask: Mask | None = None,
                             out=None, lse=None, stream=None):
    """fmha_fwd_splitkv with the partials in the library's own fixed device scratch (no
    workspace, no allocation inside the call when out / lse are given): returns (out, lse).
    Calls that overlap on one GPU race on that scratch."""
    import torch
    lib = load_library()
    B, Nq, H, _ = q.shape
    Dv = v.shape[3]
    if out is None:
        out = torch.empty((B, Nq, H, Dv), dtype=q.dtype, device=q.device)
    if lse is None:
        lse = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device)
    a, _keep = _fwd_args(q, k, v, out, lse, scale, 0.0, 0.0, mask, None)
    _check(lib.fmha_fwd_splitkv_noalloc(ctypes.byref(a), int(num_splits), _stream(stream)),
           "fmha_fwd_splitkv_noalloc")
    return out, lse


def _varlen(cu_seqlens_q, cu_seqlens_k, total_q, seqused_q, seqused_k):
    """The fmha_varlen descriptor (offsets and used lengths stay on the device)."""
    B = cu_seqlens_q.numel() - 1
    for t, n in ((seqused_q, "seqused_q"), (seqused_k, "seqused_k")):
        if t is None:
            continue
        _need_device(t, n)
        if str(t.dtype) != "torch.int32" or not t.is_contiguous() or t.dim() != 1 or t.numel() != B:
            raise ValueError(f"{n} must be a contiguous int32 [B] device tensor")
    vl = CVarlen()
    vl.cu_seqlens_q, vl.cu_seqlens_k = cu_seqlens_q.data_ptr(), cu_seqlens_k.data_ptr()
    vl.total_q, vl.reserved = total_q, 0
    vl.seqused_q = None if seqused_q is None else seqused_q.data_ptr()
    vl.seqused_k = None if seqused_k is None else seqused_k.data_ptr()
    return vl


def fmha_fwd_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q: int, max_seqlen_k: int, *,
                    scale=None, softcap=0.0, bias_slope=0.0, mask: Mask | None = None, out=None, lse=None,
                    seqused_q=None, seqused_k=None, stream=None):
    """Forward over packed variable-length sequences. q [total_q, H, Dqk], k [total_k, Hkv, Dqk],
    v [total_k, Hkv, Dv] (bf16; Hkv divides H); cu_seqlens_q / cu_seqlens_k: contiguous int32 device tensors
    [B + 1] of ascending row offsets starting at 0; max_seqlen_q / max_seqlen_k bound every
    sequence's length (the offsets are not read on the host). seqused_q / seqused_k: optional
    contiguous int32 device tensors [B]; only the first seqused[b] rows of each sequence take
    part and rows past them are left as they were in ``out`` / ``lse``. Returns
    (out [total_q, H, Dv], lse [H, total_q] fp32)."""
    import torch
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (cu_seqlens_q, "cu_seqlens_q"), (cu_seqlens_k, "cu_seqlens_k")):
        _need_device(t, n)
    if q.dim() != 3 or k.dim() != 3 or v.dim() != 3:
        raise ValueError("varlen q / k / v are [total, H, D]")
    for t in (cu_seqlens_q, cu_seqlens_k):
        if str(t.dtype) != "torch.int32" or not t.is_contiguous() or t.dim() != 1:
            raise ValueError("cu_seqlens must be contiguous int32 [B + 1] device tensors")
    if cu_seqlens_q.numel() != cu_seqlens_k.numel() or cu_seqlens_q.numel() < 2:
        raise ValueError("cu_seqlens_q and cu_seqlens_k must both hold B + 1 >= 2 offsets")
    total_q, H, _ = q.shape
    Dv = v.shape[2]
    if out is None:
        out = torch.empty((total_q, H, Dv), dtype=q.dtype, device=q.device)
    if lse is None:
        lse = torch.empty((H, total_q), dtype=torch.float32, device=q.device)
    if tuple(lse.shape) != (H, total_q) or str(lse.dtype) != "torch.float32" or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous float32 [H, total_q] tensor")
    # one-"batch" views give the seq / head strides; B, Nq, Nk are then the varlen ones
    a, _keep = _fwd_args(q.unsqueeze(0), k.unsqueeze(0), v.unsqueeze(0), out.unsqueeze(0),
                         lse.view(1, H, total_q), scale, softcap, bias_slope, mask, None)
    a.B = cu_seqlens_q.numel() - 1
    a.Nq, a.Nk = int(max_seqlen_q), int(max_seqlen_k)
    vl = _varlen(cu_seqlens_q, cu_seqlens_k, total_q, seqused_q, seqused_k)
    _check(load_library().fmha_fwd_varlen(ctypes.byref(a), ctypes.byref(vl), _stream(stream)), "fmha_fwd_varlen")
    return out, lse


def fmha_bwd_varlen(q, k, v, out, lse, dout, cu_seqlens_q, cu_seqlens_k, max_seqlen_q: int, max_seqlen_k: int, *,
                    scale=None, softcap=0.0, bias_slope=0.0, mask: Mask | None = None, dq=None, dk=None,
                    dv=None, workspace=None, seqused_q=None, seqused_k=None, stream=None):
    """Backward over packed variable-length sequences (layouts and seqused of
    fmha_fwd_varlen): returns (dq [total_q, H, Dqk], dk, dv [total_k, H, D]) in bf16; rows past
    a sequence's used length keep what the given dq / dk / dv held."""
    import torch
    lib = load_library()
    if q.dim() != 3 or k.dim() != 3 or v.dim() != 3 or out.dim() != 3 or dout.dim() != 3:
        raise ValueError("varlen tensors are [total, H, D]")
    for t in (cu_seqlens_q, cu_seqlens_k):
        _need_device(t, "cu_seqlens")
        if str(t.dtype) != "torch.int32" or not t.is_contiguous() or t.dim() != 1:
            raise ValueError("cu_seqlens must be contiguous int32 [B + 1] device tensors")
    if cu_seqlens_q.numel() != cu_seqlens_k.numel() or cu_seqlens_q.numel() < 2:
        raise ValueError("cu_seqlens_q and cu_seqlens_k must both hold B + 1 >= 2 offsets")
    total_q, H, _ = q.shape
    B = cu_seqlens_q.numel() - 1
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    need = lib.fmha_bwd_workspace_size(B, H, int(max_seqlen_q))
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    for t, n in ((dout, "dout"), (dq, "dq"), (dk, "dk"), (dv, "dv"), (workspace, "workspace")):
        _need_device(t, n)
    if dout.shape != out.shape or dq.shape != q.shape or dk.shape != k.shape or dv.shape != v.shape:
        raise ValueError("gradient shapes must match q / k / v / out")
    if tuple(lse.shape) != (H, total_q):
        raise ValueError("lse must be [H, total_q]")
    a, _keep = _fwd_args(q.unsqueeze(0), k.unsqueeze(0), v.unsqueeze(0), out.unsqueeze(0),
                         lse.view(1, H, total_q), scale, softcap, bias_slope, mask, None)
    a.B = B
    a.Nq, a.Nk = int(max_seqlen_q), int(max_seqlen_k)
    g = CBwdArgs()
    g.dout, g.dq, g.dk, g.dv = dout.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr()
    g.do_stride, g.dq_stride, g.dk_stride, g.dv_stride = (_strides(t.unsqueeze(0)) for t in (dout, dq, dk, dv))
    g.workspace = workspace.data_ptr()
    g.workspace_bytes = workspace.numel() * workspace.element_size()
    vl = _varlen(cu_seqlens_q, cu_seqlens_k, total_q, seqused_q, seqused_k)
    _check(lib.fmha_bwd_varlen(ctypes.byref(a), ctypes.byref(g), ctypes.byref(vl), _stream(stream)),
           "fmha_bwd_varlen")
    return dq, dk, dv


def splitkv_workspace_size(B, H, Nq, Dv, num_splits) -> int:
    return int(load_library().fmha_fwd_splitkv_workspace_size(B, H, Nq, Dv, num_splits))


def bwd_workspace_size(B, H, Nq) -> int:
    return int(load_library().fmha_bwd_workspace_size(B, H, Nq))


def build_block_mask(mask: Mask, B: int, Nq: int, Nk: int, tile_m: int, tile_n: int, *,
                     heads: int = 1, device="cuda", stream=None) -> BlockSparse:
    """Classify every (tile_m x tile_n) tile of the element mask on the GPU and return
    the forward and transposed index lists."""
    import torch
    nqt, nkt = -(-Nq // tile_m), -(-Nk // tile_n)
    # the eight arrays are contiguous slices of one allocation (one allocator call per build)
    shapes = [(B, heads, nqt), (B, heads, nqt, nkt), (B, heads, nqt), (B, heads, nqt, nkt),
              (B, heads, nkt), (B, heads, nkt, nqt), (B, heads, nkt), (B, heads, nkt, nqt)]
    sizes = [math.prod(sh) for sh in shapes]
    flat = torch.empty(sum(sizes), dtype=torch.int32, device=device)
    parts, o = [], 0
    for sh, n in zip(shapes, sizes):
        parts.append(flat[o:o + n].view(sh))
        o += n
    bs = BlockSparse(tile_m, tile_n, nqt, nkt, heads, *parts)
    c = bs.to_c()
    cm = mask.to_c()
    _check(load_library().build_block_mask(ctypes.byref(cm), B, heads, Nq, Nk, tile_m, tile_n,
                                           ctypes.byref(c), _stream(stream)), "build_block_mask")
    return bs
