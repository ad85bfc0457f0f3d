"""Element mask predicates (oracle; test infrastructure only).

Index convention: i is the absolute query row, j the absolute key column, and
delta = Nk - Nq. The pages name the mask kinds without printing their definitions
([2CTA] "Testing Testing Testing", the fuzz tester's case lists and mask names), so the
readings below are the plainest ones consistent with the rest of the pages:

  none            always allowed
  causal          j <= i + delta            (bottom-right aligned: a single decode query
                                             sees every key; equals top-left when Nq = Nk)
  sliding_window  i + delta - W <= j <= i + delta   (both ends inclusive, no right context)
  block_diagonal  doc_q[i] == doc_k[j]      (no causal restriction inside a document)
  prefix_lm       j < P  or  j <= i + delta (bidirectional prefix, causal after it)

The window width used by the fuzz tester is max(64, min(Nq, Nk) // 3)
([2CTA] "Testing Testing Testing", window_size) -- provided here as ``fuzz_window``.

Block-sparse semantics ([2CTA] "Summary" and the fuzz tester's block_sparse_tensors):
a (tile_m x tile_n) tile listed as FULL is allowed everywhere, a tile listed as PARTIAL
applies the element predicate, and an unlisted tile is skipped entirely.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

KINDS = ("none", "causal", "sliding_window", "block_diagonal", "prefix_lm")


@dataclass
class MaskSpec:
    kind: str = "none"
    window: int = 0          # W for sliding_window
    prefix: int = 0          # P for prefix_lm
    doc_q: np.ndarray | None = field(default=None, repr=False)  # [B, Nq] int
    doc_k: np.ndarray | None = field(default=None, repr=False)  # [B, Nk] int

    def __post_init__(self):
        if self.kind not in KINDS:
            raise ValueError(f"unknown mask kind {self.kind!r}")
        if self.kind == "block_diagonal" and (self.doc_q is None or self.doc_k is None):
            raise ValueError("block_diagonal needs doc_q and doc_k")


def fuzz_window(nq: int, nk: int) -> int:
    return max(64, min(nq, nk) // 3)


def allowed(mask: MaskSpec, b: int, qidx, kidx, nq: int, nk: int) -> np.ndarray:
    """Boolean [len(qidx), len(kidx)]: is key kidx[c] visible from query qidx[r]."""
    i = np.asarray(qidx, dtype=np.int64)[:, None]
    j = np.asarray(kidx, dtype=np.int64)[None, :]
    delta = nk - nq
    if mask.kind == "none":
        return np.ones((i.shape[0], j.shape[1]), dtype=bool)
    if mask.kind == "causal":
        return j <= i + delta
    if mask.kind == "sliding_window":
        return (j <= i + delta) & (j >= i + delta - mask.window)
    if mask.kind == "block_diagonal":
        dq = np.asarray(mask.doc_q[b], dtype=np.int64)[i[:, 0]][:, None]
        dk = np.asarray(mask.doc_k[b], dtype=np.int64)[j[0, :]][None, :]
        return dq == dk
    if mask.kind == "prefix_lm":
        return (j < mask.prefix) | (j <= i + delta)
    raise AssertionError(mask.kind)


def tile_sets(lists, b: int, hm: int):
    """The listed tiles of mask head ``hm`` as two boolean [nQt, nKt] sets (full,
    partial). Each row holds ``cnt`` entries (a count below 0 reads as 0, above the
    row length as the whole row); an entry is a key-tile index, and an index outside
    [0, nKt) names no tile, so it adds nothing. Membership is set membership: an entry
    given twice is one entry."""
    n_qt, n_kt = lists.partial_idx.shape[2], lists.partial_idx.shape[3]
    is_full = np.zeros((n_qt, n_kt), dtype=bool)
    is_part = np.zeros((n_qt, n_kt), dtype=bool)
    for dst, cnt, idx in ((is_full, lists.full_cnt, lists.full_idx),
                          (is_part, lists.partial_cnt, lists.partial_idx)):
        for r in range(n_qt):
            c = min(max(int(cnt[b, hm, r]), 0), n_kt)
            for t in idx[b, hm, r, :c]:
                if 0 <= t < n_kt:
                    dst[r, t] = True
    return is_full, is_part


def block_sparse_allowed(lists, mask: MaskSpec, b: int, h: int, qidx, kidx,
                         nq: int, nk: int) -> np.ndarray:
    """Element visibility under block-sparse index lists (forward lists of ``lists``):
    full tiles are visible everywhere, partial tiles apply ``mask``, others are skipped.
    A tile listed both as full and as partial is full (its full listing makes every
    element visible; the partial listing only adds elements the mask allows). Lists
    with one mask head serve every attention head; otherwise head h reads mask head h."""
    hm = h if lists.partial_cnt.shape[1] > 1 else 0
    qt = np.asarray(qidx, dtype=np.int64) // lists.tile_m
    kt = np.asarray(kidx, dtype=np.int64) // lists.tile_n
    is_full, is_part = tile_sets(lists, b, hm)
    full = is_full[qt[:, None], kt[None, :]]
    part = is_part[qt[:, None], kt[None, :]]
    return full | (part & allowed(mask, b, qidx, kidx, nq, nk))
