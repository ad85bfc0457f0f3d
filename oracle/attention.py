"""Materialised fp64 attention: forward, backward, split-KV partials and combine.

TEST INFRASTRUCTURE ONLY (see the package docstring). Layouts follow the fuzz tester
of [2CTA] ("Testing Testing Testing", create_tensors / _flash_attn_fwd): Q, K, V, O, dO
are BSHD ``[batch, seq, head, dim]``; LSE is ``[batch, head, seq_q]``.

Definition (per batch b, head h), following the math-backend formula of [SDPA]
(attn_weight = Q K^T * scale, softmax over keys, times V) extended with the terms the
fuzz tester passes to the kernels ([2CTA]: softmax_scale = 1/sqrt(headdim), softcap,
score_mod = relative bias, mask_mod, return_lse):

  S_pre[i,j] = scale * <q_i, k_j>
  S[i,j]     = c * tanh(S_pre[i,j] / c)        if softcap c > 0, else S_pre[i,j]
             + sigma * |i - j|                  (relative-bias score mod; sigma may be 0)
  S[i,j]     = -inf where key j is not visible from query i
  m_i        = max_j S[i,j]
  P[i,j]     = exp(S[i,j] - m_i),  l_i = sum_j P[i,j]
  O_i        = sum_j P[i,j] v_j / l_i,  LSE_i = m_i + ln l_i
  A row with no visible key has O_i = 0 and LSE_i = -inf.

The backward recomputes P from LSE (the fuzz tester's backward takes out, dout and lse):
  P = exp(S - LSE) (0 where masked), dV = P^T dO, dP = dO V^T,
  D_i = sum_j P[i,j] dP[i,j], dS = P * (dP - D), times 1 - tanh^2(S_pre/c) under softcap
  (the bias has no learnable input, so its gradient passes straight through: the
  fuzz tester's score_mod_bwd_rel_bias returns grad unchanged),
  dQ = scale * dS K, dK = scale * dS^T Q.

Split-KV ([FDMA] "Testing": split-KV multi-splits 1,2,4,8,16): each split attends to a
contiguous key range and returns its own normalised (O_s, LSE_s); the combine is the
two-chunk merge rule of [SDPA] applied over all splits:
  LSE = ln sum_s exp(LSE_s),  O = sum_s exp(LSE_s - LSE) O_s.
"""
from __future__ import annotations

import math

import numpy as np

from .masks import MaskSpec, allowed, block_sparse_allowed


def _f64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


def default_scale(dqk: int) -> float:
    return 1.0 / math.sqrt(dqk)


def visible(mask: MaskSpec, lists, b, h, qidx, kidx, nq, nk) -> np.ndarray:
    if lists is None:
        return allowed(mask, b, qidx, kidx, nq, nk)
    return block_sparse_allowed(lists, mask, b, h, qidx, kidx, nq, nk)


def scores_bh(q_rows, k, qidx, kidx, scale, softcap=0.0, bias_slope=0.0):
    """Return (S without mask, S_pre) for the given query rows and keys, fp64."""
    s_pre = scale * (_f64(q_rows) @ _f64(k).T)
    s = softcap * np.tanh(s_pre / softcap) if softcap > 0 else s_pre.copy()
    if bias_slope != 0.0:
        i = np.asarray(qidx, dtype=np.int64)[:, None]
        j = np.asarray(kidx, dtype=np.int64)[None, :]
        s = s + bias_slope * np.abs(i - j).astype(np.float64)
    return s, s_pre


def _softmax_rows(s, vis):
    """Masked softmax pieces: (P unnormalised, m, l, empty-row flags)."""
    s = np.where(vis, s, -np.inf)
    empty = ~vis.any(axis=1)
    m = np.where(empty, 0.0, s.max(axis=1, initial=-np.inf))
    p = np.where(vis, np.exp(s - m[:, None]), 0.0)
    l = p.sum(axis=1)
    return p, m, l, empty


def forward_bh(q_rows, k, v, qidx, b, h, nq, nk, *, scale, softcap=0.0, bias_slope=0.0,
               mask: MaskSpec = MaskSpec(), lists=None, kidx=None):
    """Forward for one (b, h) over the given query rows (absolute indices ``qidx``)
    and the keys ``k``/``v`` whose absolute indices are ``kidx`` (default 0..Nk-1).
    Returns (O rows, LSE rows)."""
    if kidx is None:
        kidx = np.arange(nk)
    k = _f64(k)
    v = _f64(v)
    s, _ = scores_bh(q_rows, k, qidx, kidx, scale, softcap, bias_slope)
    vis = visible(mask, lists, b, h, qidx, kidx, nq, nk)
    p, m, l, empty = _softmax_rows(s, vis)
    safe_l = np.where(empty, 1.0, l)
    o = (p @ v) / safe_l[:, None]
    o[empty] = 0.0
    lse = np.where(empty, -np.inf, m + np.log(safe_l))
    return o, lse


def kv_head(h: int, H: int, Hkv: int) -> int:
    """K/V head read by query head h when H query heads share Hkv K/V heads (grouped-query
    attention, as in the reference call with ``enable_gqa=True`` and separate query and
    key/value head counts of "Enable 2CTA for SM100 block-sparse backward", section
    "Testing Testing Testing"): consecutive groups of H / Hkv query heads share one K/V
    head. Hkv = H is multi-head attention, Hkv = 1 multi-query attention."""
    if Hkv < 1 or H % Hkv != 0:
        raise ValueError(f"{H} query heads cannot share {Hkv} key/value heads")
    return h // (H // Hkv)


def forward(q, k, v, *, scale=None, softcap=0.0, bias_slope=0.0, mask: MaskSpec = MaskSpec(),
            lists=None, heads=None, rows=None):
    """Full forward. q [B,Nq,H,Dqk], k [B,Nk,Hkv,Dqk], v [B,Nk,Hkv,Dv] (Hkv divides H;
    query head h reads K/V head kv_head(h, H, Hkv)).

    ``heads``/``rows`` restrict the computation to a subset (the rest of the output is
    NaN), for sampled comparisons at sizes where the full product is too large."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, nq, H, dqk = q.shape
    nk, dv = k.shape[1], v.shape[3]
    hkv = k.shape[2]
    if v.shape[2] != hkv:
        raise ValueError("k and v must have the same number of heads")
    scale = default_scale(dqk) if scale is None else scale
    heads = range(H) if heads is None else heads
    qidx = np.arange(nq) if rows is None else np.asarray(rows, dtype=np.int64)
    o = np.full((B, nq, H, dv), np.nan)
    lse = np.full((B, H, nq), np.nan)
    for b in range(B):
        for h in heads:
            g = kv_head(h, H, hkv)
            ob, lb = forward_bh(q[b, qidx, h], k[b, :, g], v[b, :, g], qidx, b, h, nq, nk,
                                scale=scale, softcap=softcap, bias_slope=bias_slope,
                                mask=mask, lists=lists)
            o[b, qidx, h] = ob
            lse[b, h, qidx] = lb
    return o, lse


def used_rows(cu, seqused, b: int) -> int:
    """Rows of sequence b that take part: its whole span cu[b]:cu[b+1], or the first
    seqused[b] of them (the forward's seqused_q / seqused_k arguments of "Enable 2CTA for
    SM100 block-sparse backward", section "Testing Testing Testing", passed there without a
    definition; read here as the used prefix of each span)."""
    span = int(cu[b + 1]) - int(cu[b])
    if seqused is None:
        return span
    u = int(seqused[b])
    if not 0 <= u <= span:
        raise ValueError(f"seqused[{b}] = {u} outside [0, {span}]")
    return u


def forward_varlen(q, k, v, cu_q, cu_k, *, scale=None, softcap=0.0, bias_slope=0.0,
                   mask: MaskSpec = MaskSpec(), seqused_q=None, seqused_k=None):
    """Packed variable-length sequences (the forward's cu_seqlens arguments of "Enable 2CTA
    for SM100 block-sparse backward", section "Testing Testing Testing"): q [total_q,H,Dqk],
    k [total_k,H,Dqk], v [total_k,H,Dv]; sequence b is query rows cu_q[b]:cu_q[b+1] and key
    rows cu_k[b]:cu_k[b+1], attended as its own batch entry (positions, masks and the
    relative bias are sequence-local). With seqused_q / seqused_k only the first rows of
    each span take part (see used_rows); rows past them are not part of the result and
    come back as NaN. Returns o [total_q,H,Dv], lse [H,total_q]."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    total_q, H, dqk = q.shape
    dv = v.shape[2]
    scale = default_scale(dqk) if scale is None else scale
    o = np.zeros((total_q, H, dv))
    lse = np.full((H, total_q), -np.inf)
    for b in range(len(cu_q) - 1):
        qs, ks = int(cu_q[b]), int(cu_k[b])
        qe, ke = qs + used_rows(cu_q, seqused_q, b), ks + used_rows(cu_k, seqused_k, b)
        o[qe:int(cu_q[b + 1])] = np.nan
        lse[:, qe:int(cu_q[b + 1])] = np.nan
        if qe == qs:
            continue
        if ke == ks:   # no keys: every row is fully masked
            continue
        ob, lb = forward(q[None, qs:qe], k[None, ks:ke], v[None, ks:ke], scale=scale, softcap=softcap,
                         bias_slope=bias_slope, mask=mask)
        o[qs:qe] = ob[0]
        lse[:, qs:qe] = lb[0]
    return o, lse


def backward_varlen(q, k, v, do, cu_q, cu_k, *, scale=None, softcap=0.0, bias_slope=0.0,
                    mask: MaskSpec = MaskSpec(), seqused_q=None, seqused_k=None):
    """Backward of forward_varlen: each sequence as its own batch entry (the batched
    backward on its used rows). Returns dq [total_q,H,Dqk], dk, dv [total_k,H,D], o, lse
    [H,total_q]; rows of sequences without keys (or queries) get zero gradients, rows past
    a used length are NaN (not part of the result)."""
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    total_q, H, dqk = q.shape
    scale = default_scale(dqk) if scale is None else scale
    dq, dk, dv = np.zeros(q.shape), np.zeros(k.shape), np.zeros(v.shape)
    o = np.zeros((total_q, H, v.shape[2]))
    lse = np.full((H, total_q), -np.inf)
    for b in range(len(cu_q) - 1):
        qs, ks = int(cu_q[b]), int(cu_k[b])
        qe, ke = qs + used_rows(cu_q, seqused_q, b), ks + used_rows(cu_k, seqused_k, b)
        for arr in (dq, o):
            arr[qe:int(cu_q[b + 1])] = np.nan
        lse[:, qe:int(cu_q[b + 1])] = np.nan
        dk[ke:int(cu_k[b + 1])] = np.nan
        dv[ke:int(cu_k[b + 1])] = np.nan
        if qe == qs or ke == ks:
            continue
        gq, gk, gv, ob, lb = backward(q[None, qs:qe], k[None, ks:ke], v[None, ks:ke], do[None, qs:qe], scale=scale,
                                      softcap=softcap, bias_slope=bias_slope, mask=mask)
        dq[qs:qe], dk[ks:ke], dv[ks:ke] = gq[0], gk[0], gv[0]
        o[qs:qe], lse[:, qs:qe] = ob[0], lb[0]
    return dq, dk, dv, o, lse


def backward_bh(q, k, v, do, b, h, *, scale, softcap=0.0, bias_slope=0.0,
                mask: MaskSpec = MaskSpec(), lists=None, lse=None):
    """Backward for one (b, h), all rows. Recomputes P from LSE (the oracle's own LSE
    unless one is given). Returns (dq, dk, dv, o, lse)."""
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    nq, nk = q.shape[0], k.shape[0]
    qidx, kidx = np.arange(nq), np.arange(nk)
    o, own_lse = forward_bh(q, k, v, qidx, b, h, nq, nk, scale=scale, softcap=softcap,
                            bias_slope=bias_slope, mask=mask, lists=lists)
    lse = own_lse if lse is None else _f64(lse)
    s, s_pre = scores_bh(q, k, qidx, kidx, scale, softcap, bias_slope)
    vis = visible(mask, lists, b, h, qidx, kidx, nq, nk)
    live = vis & np.isfinite(lse)[:, None]
    p = np.where(live, np.exp(np.where(live, s, 0.0) - np.where(np.isfinite(lse), lse, 0.0)[:, None]), 0.0)
    dv = p.T @ do
    dp = do @ v.T
    d = (p * dp).sum(axis=1)
    ds = p * (dp - d[:, None])
    if softcap > 0:
        ds = ds * (1.0 - np.tanh(s_pre / softcap) ** 2)
    dq = scale * (ds @ k)
    dk = scale * (ds.T @ q)
    return dq, dk, dv, o, lse


def backward(q, k, v, do, *, scale=None, softcap=0.0, bias_slope=0.0,
             mask: MaskSpec = MaskSpec(), lists=None, heads=None):
    """Full backward: returns dQ, dK, dV (BSHD, fp64), O and LSE of the oracle forward;
    K / V may have fewer heads than Q (see kv_head).
    ``heads`` restricts the computation (other heads are NaN)."""
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    B, nq, H, dqk = q.shape
    nk, dv_ = k.shape[1], v.shape[3]
    hkv = k.shape[2]
    if hkv != H:
        # grouped K/V heads (see kv_head): the forward is the multi-head forward on K/V
        # repeated H / Hkv times along the head axis, so a shared head's gradient is the
        # sum of its copies' gradients
        kv_head(0, H, hkv)   # validates the grouping
        G = H // hkv
        dq, dkr, dvr, o, lse = backward(q, np.repeat(k, G, axis=2), np.repeat(v, G, axis=2), do, scale=scale,
                                        softcap=softcap, bias_slope=bias_slope, mask=mask, lists=lists,
                                        heads=heads)
        return (dq, dkr.reshape(B, nk, hkv, G, dqk).sum(axis=3), dvr.reshape(B, nk, hkv, G, dv_).sum(axis=3),
                o, lse)
    scale = default_scale(dqk) if scale is None else scale
    heads = range(H) if heads is None else heads
    dq = np.full(q.shape, np.nan)
    dk = np.full(k.shape, np.nan)
    dv = np.full(v.shape, np.nan)
    o = np.full((B, nq, H, dv_), np.nan)
    lse = np.full((B, H, nq), np.nan)
    for b in range(B):
        for h in heads:
            r = backward_bh(q[b, :, h], k[b, :, h], v[b, :, h], do[b, :, h], b, h,
                            scale=scale, softcap=softcap, bias_slope=bias_slope,
                            mask=mask, lists=lists)
            dq[b, :, h], dk[b, :, h], dv[b, :, h], o[b, :, h], lse[b, h] = r
    return dq, dk, dv, o, lse


def split_ranges(nk: int, splits: int, tile_n: int):
    """Contiguous, tile-aligned key ranges: ceil(ceil(Nk/tile_n)/splits) tiles each.
    Trailing splits may be empty."""
    n_tiles = -(-nk // tile_n)
    per = -(-n_tiles // splits)
    out = []
    for s in range(splits):
        lo = min(nk, s * per * tile_n)
        hi = min(nk, (s + 1) * per * tile_n)
        out.append((lo, hi))
    return out


def split_partials(q, k, v, splits, tile_n, *, scale=None, softcap=0.0, bias_slope=0.0,
                   mask: MaskSpec = MaskSpec()):
    """Per-split normalised partial outputs: list of (O_s [B,Nq,H,Dv], LSE_s [B,H,Nq]).
    An empty split (or a row with no visible key in the split) gives O_s = 0,
    LSE_s = -inf. K/V may have fewer heads than Q (see kv_head)."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, nq, H, dqk = q.shape
    nk, dv = k.shape[1], v.shape[3]
    hkv = k.shape[2]
    scale = default_scale(dqk) if scale is None else scale
    qidx = np.arange(nq)
    parts = []
    for lo, hi in split_ranges(nk, splits, tile_n):
        o = np.zeros((B, nq, H, dv))
        lse = np.full((B, H, nq), -np.inf)
        if hi > lo:
            kidx = np.arange(lo, hi)
            for b in range(B):
                for h in range(H):
                    g = kv_head(h, H, hkv)
                    s, _ = scores_bh(q[b, :, h], k[b, lo:hi, g], qidx, kidx, scale, softcap, bias_slope)
                    vis = allowed(mask, b, qidx, kidx, nq, nk)
                    p, m, l, empty = _softmax_rows(s, vis)
                    safe_l = np.where(empty, 1.0, l)
                    ob = (p @ v[b, lo:hi, g]) / safe_l[:, None]
                    ob[empty] = 0.0
                    o[b, :, h] = ob
                    lse[b, h] = np.where(empty, -np.inf, m + np.log(safe_l))
        parts.append((o, lse))
    return parts


def combine_partials(parts):
    """LSE-weighted combine of normalised partials (merge rule of [SDPA])."""
    lses = np.stack([p[1] for p in parts])            # [S, B, H, Nq]
    outs = np.stack([p[0] for p in parts])            # [S, B, Nq, H, Dv]
    mx = lses.max(axis=0)
    empty = ~np.isfinite(mx)
    mx_safe = np.where(empty, 0.0, mx)
    w = np.exp(lses - mx_safe[None])                  # exp(-inf) = 0 for empty splits
    tot = w.sum(axis=0)
    lse = np.where(empty, -np.inf, mx_safe + np.log(np.where(empty, 1.0, tot)))
    wn = w / np.where(empty, 1.0, tot)[None]          # [S, B, H, Nq]
    o = np.einsum("sbhq,sbqhd->bqhd", wn, outs)
    return o, lse


def streaming_forward_bh(q_rows, k, v, qidx, b, h, nq, nk, tile_n, *, scale, softcap=0.0,
                         bias_slope=0.0, mask: MaskSpec = MaskSpec()):
    """The same forward computed by streaming key tiles with the running (m, l, o)
    merge of [SDPA] (a cross-check of the materialised definition, in fp64)."""
    q_rows, k, v = _f64(q_rows), _f64(k), _f64(v)
    r = q_rows.shape[0]
    m = np.full(r, -np.inf)
    l = np.zeros(r)
    o = np.zeros((r, v.shape[1]))
    for lo in range(0, nk, tile_n):
        hi = min(nk, lo + tile_n)
        kidx = np.arange(lo, hi)
        s, _ = scores_bh(q_rows, k[lo:hi], qidx, kidx, scale, softcap, bias_slope)
        vis = allowed(mask, b, qidx, kidx, nq, nk)
        s = np.where(vis, s, -np.inf)
        m_tile = s.max(axis=1)
        m_new = np.maximum(m, m_tile)
        live = np.isfinite(m_new)
        m_use = np.where(live, m_new, 0.0)
        corr = np.where(np.isfinite(m), np.exp(m - m_use), 0.0)
        p = np.where(vis, np.exp(s - m_use[:, None]), 0.0)
        l = corr * l + p.sum(axis=1)
        o = corr[:, None] * o + p @ v[lo:hi]
        m = m_new
    empty = l == 0.0
    out = np.where(empty[:, None], 0.0, o / np.where(empty, 1.0, l)[:, None])
    lse = np.where(empty, -np.inf, m + np.log(np.where(empty, 1.0, l)))
    return out, lse
