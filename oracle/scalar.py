"""Pure-Python scalar brute force for tiny shapes (N <= 16, D <= 8).

TEST INFRASTRUCTURE ONLY. An independent second formulation of the same definition as
``attention`` (math-backend softmax(Q K^T * scale) V of [SDPA], with the score terms of
[2CTA]'s fuzz tester), written with Python floats, ``math.exp`` and ``math.fsum`` and its
own mask predicates, so that a slip in the vectorised oracle shows up as a mismatch.
"""
from __future__ import annotations

import math


def _visible(kind, i, j, nq, nk, window=0, prefix=0, doc_q=None, doc_k=None):
    d = nk - nq
    if kind == "none":
        return True
    if kind == "causal":
        return j - i <= d
    if kind == "sliding_window":
        return i + d - window <= j <= i + d
    if kind == "block_diagonal":
        return doc_q[i] == doc_k[j]
    if kind == "prefix_lm":
        return j < prefix or j - d <= i
    raise ValueError(kind)


def _score(qi, kj, i, j, scale, softcap, slope):
    x = scale * math.fsum(a * b for a, b in zip(qi, kj))
    if softcap > 0:
        x = softcap * math.tanh(x / softcap)
    return x + slope * abs(i - j)


def attend(q, k, v, scale, kind="none", softcap=0.0, slope=0.0, **mk):
    """q: list of Nq rows, k: Nk rows, v: Nk rows. Returns (O rows, LSE list)."""
    nq, nk = len(q), len(k)
    outs, lses = [], []
    for i in range(nq):
        sc = {}
        for j in range(nk):
            if _visible(kind, i, j, nq, nk, **mk):
                sc[j] = _score(q[i], k[j], i, j, scale, softcap, slope)
        if not sc:
            outs.append([0.0] * len(v[0]))
            lses.append(-math.inf)
            continue
        top = max(sc.values())
        w = {j: math.exp(s - top) for j, s in sc.items()}
        tot = math.fsum(w.values())
        outs.append([math.fsum(w[j] * v[j][c] for j in w) / tot for c in range(len(v[0]))])
        lses.append(top + math.log(tot))
    return outs, lses


def attend_grad(q, k, v, do, scale, kind="none", softcap=0.0, slope=0.0, **mk):
    """Gradients of sum(O * dO) w.r.t. q, k, v by the chain rule, element by element."""
    nq, nk, dq_, dv_ = len(q), len(k), len(q[0]), len(v[0])
    _, lse = attend(q, k, v, scale, kind, softcap, slope, **mk)
    gq = [[0.0] * dq_ for _ in range(nq)]
    gk = [[0.0] * dq_ for _ in range(nk)]
    gv = [[0.0] * dv_ for _ in range(nk)]
    for i in range(nq):
        if lse[i] == -math.inf:
            continue
        p = {}
        for j in range(nk):
            if _visible(kind, i, j, nq, nk, **mk):
                p[j] = math.exp(_score(q[i], k[j], i, j, scale, softcap, slope) - lse[i])
        dp = {j: math.fsum(do[i][c] * v[j][c] for c in range(dv_)) for j in p}
        dd = math.fsum(p[j] * dp[j] for j in p)
        for j in p:
            g = p[j] * (dp[j] - dd)
            if softcap > 0:
                raw = scale * math.fsum(a * b for a, b in zip(q[i], k[j]))
                g *= 1.0 - math.tanh(raw / softcap) ** 2
            for c in range(dq_):
                gq[i][c] += scale * g * k[j][c]
                gk[j][c] += scale * g * q[i][c]
            for c in range(dv_):
                gv[j][c] += p[j] * do[i][c]
    return gq, gk, gv
