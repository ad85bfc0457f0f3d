"""Block-sparse tile classification and index lists, by element enumeration.

TEST INFRASTRUCTURE ONLY. Follows the block-sparse construction the fuzz tester of
[2CTA] performs before each launch ("Testing Testing Testing":
_build_block_sparse_masks_for_bwd builds forward lists per query tile and separate
backward lists per key tile from an element mask_mod, with the sparse tile size
decoupled from the kernel tile). Every in-bounds element of every tile is evaluated;
the predicate is never evaluated out of bounds.

  empty   : no in-bounds element of the tile is visible
  full    : every in-bounds element is visible
  partial : otherwise

List layout (a reading; the pages do not print one): for each (b, mask head, query
tile) a count and the ascending key-tile indices, padded with -1 to the number of key
tiles; separately for partial and full tiles. The transposed (backward) lists are the
same per key tile over query tiles.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from .masks import MaskSpec, allowed

EMPTY, PARTIAL, FULL = 0, 1, 2


@dataclass
class BlockLists:
    tile_m: int
    tile_n: int
    partial_cnt: np.ndarray    # [B, Hm, nQt] int32
    partial_idx: np.ndarray    # [B, Hm, nQt, nKt] int32, -1 padded
    full_cnt: np.ndarray
    full_idx: np.ndarray
    t_partial_cnt: np.ndarray  # [B, Hm, nKt]
    t_partial_idx: np.ndarray  # [B, Hm, nKt, nQt]
    t_full_cnt: np.ndarray
    t_full_idx: np.ndarray


def classify_tiles(mask: MaskSpec, B: int, Hm: int, nq: int, nk: int, tile_m: int,
                   tile_n: int) -> np.ndarray:
    """Tile classes [B, Hm, nQt, nKt] in {EMPTY, PARTIAL, FULL}."""
    n_qt, n_kt = -(-nq // tile_m), -(-nk // tile_n)
    cls = np.zeros((B, Hm, n_qt, n_kt), dtype=np.int8)
    for b in range(B):
        for r in range(n_qt):
            qidx = np.arange(r * tile_m, min(nq, (r + 1) * tile_m))
            row_vis = allowed(mask, b, qidx, np.arange(nk), nq, nk)  # in-bounds only
            for c in range(n_kt):
                blk = row_vis[:, c * tile_n: min(nk, (c + 1) * tile_n)]
                n_vis = int(blk.sum())
                if n_vis == 0:
                    k = EMPTY
                elif n_vis == blk.size:
                    k = FULL
                else:
                    k = PARTIAL
                cls[b, :, r, c] = k   # the mask kinds here do not depend on the head
    return cls


def _lists(cls2d: np.ndarray, want: int):
    rows, cols = cls2d.shape
    cnt = np.zeros(rows, dtype=np.int32)
    idx = np.full((rows, cols), -1, dtype=np.int32)
    for r in range(rows):
        sel = np.nonzero(cls2d[r] == want)[0]
        cnt[r] = len(sel)
        idx[r, : len(sel)] = sel
    return cnt, idx


def build_lists(mask: MaskSpec, B: int, Hm: int, nq: int, nk: int, tile_m: int,
                tile_n: int) -> BlockLists:
    cls = classify_tiles(mask, B, Hm, nq, nk, tile_m, tile_n)
    n_qt, n_kt = cls.shape[2], cls.shape[3]
    pc = np.zeros((B, Hm, n_qt), np.int32); pi = np.full((B, Hm, n_qt, n_kt), -1, np.int32)
    fc = np.zeros((B, Hm, n_qt), np.int32); fi = np.full((B, Hm, n_qt, n_kt), -1, np.int32)
    tpc = np.zeros((B, Hm, n_kt), np.int32); tpi = np.full((B, Hm, n_kt, n_qt), -1, np.int32)
    tfc = np.zeros((B, Hm, n_kt), np.int32); tfi = np.full((B, Hm, n_kt, n_qt), -1, np.int32)
    for b in range(B):
        for h in range(Hm):
            c = cls[b, h]
            pc[b, h], pi[b, h] = _lists(c, PARTIAL)
            fc[b, h], fi[b, h] = _lists(c, FULL)
            tpc[b, h], tpi[b, h] = _lists(c.T, PARTIAL)
            tfc[b, h], tfi[b, h] = _lists(c.T, FULL)
    return BlockLists(tile_m, tile_n, pc, pi, fc, fi, tpc, tpi, tfc, tfi)
