"""Seeded synthetic inputs shared by the tests, the benchmark and the oracle checks.

This module generates data only: it holds none of the attention arithmetic. Both the
HIP path and the CPU oracle consume exactly the arrays produced here, so a parity test
never depends on two random generators agreeing.

Recipe (stated once, used everywhere):
  * generator: ``numpy.random.default_rng(seed)`` (PCG64);
  * tensors are drawn with ``standard_normal(dtype=float32)`` in the order the caller
    lists them, each in BSHD order ``[batch, seq, head, dim]``;
  * bf16 inputs are the fp32 draws rounded to nearest-even on the fp32 bit pattern;
  * document lengths for block-diagonal masks are integers uniform on
    ``[lo, hi]`` drawn until their running sum reaches the sequence length, the last
    one truncated to fit, per batch element in order, from a generator seeded
    ``1000 + seed``.
"""
from __future__ import annotations

import numpy as np

BASE_SEED = 42


def case_seed(config: int, case: int = 0) -> int:
    """Seed of case ``case`` of workload group ``config``: 42 + 1000*config + case."""
    return BASE_SEED + 1000 * config + case


def bf16_bits(x: np.ndarray, chunk: int = 1 << 24) -> np.ndarray:
    """Round fp32 values to bf16 (round to nearest, ties to even); return the uint16 bits.
    Works in chunks so that very large tensors need little temporary memory."""
    flat = np.ascontiguousarray(x, dtype=np.float32).reshape(-1).view(np.uint32)
    out = np.empty(flat.shape, dtype=np.uint16)
    for lo in range(0, flat.size, chunk):
        u = flat[lo:lo + chunk].astype(np.uint64)
        out[lo:lo + chunk] = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    return out.reshape(np.shape(x))


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to fp32."""
    return (bits.astype(np.uint32) << 16).view(np.float32)


class Tensor:
    """One synthetic tensor: its values as fp32 (exactly the values the kernels see) and,
    for bf16, the raw bit pattern to upload."""

    def __init__(self, values: np.ndarray, bits: np.ndarray | None, dtype: str):
        self.values = values  # float32 array, exact
        self.bits = bits      # uint16 array for bf16, None for fp32
        self.dtype = dtype

    @property
    def shape(self):
        return self.values.shape

    def to_torch(self, device="cpu"):
        import torch
        if self.dtype == "bf16":
            t = torch.from_numpy(self.bits.view(np.int16).copy()).view(torch.bfloat16)
        else:
            t = torch.from_numpy(self.values.copy())
        return t.to(device)


def normal_tensors(seed: int, shapes, dtype: str = "bf16"):
    """Draw iid N(0,1) tensors of the given shapes, in order, from one generator."""
    if dtype not in ("bf16", "fp32"):
        raise ValueError(dtype)
    rng = np.random.default_rng(seed)
    out = []
    for shp in shapes:
        x = rng.standard_normal(size=tuple(shp), dtype=np.float32)
        if dtype == "bf16":
            bits = bf16_bits(x)
            out.append(Tensor(bf16_bits_to_f32(bits), bits, "bf16"))
        else:
            out.append(Tensor(x, None, "fp32"))
    return out


def attention_inputs(seed: int, B: int, Nq: int, Nk: int, H: int, Dqk: int, Dv: int,
                     dtype: str = "bf16", with_dout: bool = False):
    """Q [B,Nq,H,Dqk], K [B,Nk,H,Dqk], V [B,Nk,H,Dv] (and dO [B,Nq,H,Dv]) in that order."""
    shapes = [(B, Nq, H, Dqk), (B, Nk, H, Dqk), (B, Nk, H, Dv)]
    if with_dout:
        shapes.append((B, Nq, H, Dv))
    return normal_tensors(seed, shapes, dtype)


def document_ids(seed: int, B: int, N: int, lo: int = 256, hi: int = 2048) -> np.ndarray:
    """Document id per token, int32 [B, N]; ids count up from 0 within each batch row."""
    rng = np.random.default_rng(1000 + seed)
    ids = np.empty((B, N), dtype=np.int32)
    for b in range(B):
        pos, doc = 0, 0
        while pos < N:
            length = int(rng.integers(lo, hi, endpoint=True))
            end = min(N, pos + length)
            ids[b, pos:end] = doc
            pos, doc = end, doc + 1
    return ids
