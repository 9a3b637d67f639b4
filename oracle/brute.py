"""Pure-Python scalar-loop attention for tiny inputs (N <= 16) -- test infrastructure only.

No numpy arithmetic: every sum is ``math.fsum`` (exactly rounded) and every
exponential is ``math.exp``. It exists to pin ``oracle.attention`` on small
cases, including the backward, by an independent evaluation order.
"""
from __future__ import annotations

import math


def _dot(a, b):
    return math.fsum(x * y for x, y in zip(a, b))


def _keys(i, n_q, n_k, causal, window, block_mask=None, block=128):
    """Keys row i keeps: from i + (n_k - n_q) - window (or 0) up to i + (n_k - n_q) (or the last key),
    and, with a block mask (nested lists of bools), only those whose (i // block, j // block) entry is true."""
    diag = i + n_k - n_q
    first = max(0, diag - window) if window >= 0 else 0
    last = min(n_k - 1, diag) if causal else n_k - 1
    return [j for j in range(first, last + 1) if block_mask is None or block_mask[i // block][j // block]]


def forward(q, k, v, causal, scale, window=-1, block_mask=None, block=128):
    """q: nested list [N_q][D], k, v: [N_k][D] floats for one head. Returns (O [N_q][D], lse [N_q])."""
    n = len(q)
    o, lse = [], []
    for i in range(n):
        keys = _keys(i, n, len(k), causal, window, block_mask, block)
        if not keys:  # a row that keeps no key: empty sum, lse = ln 0, output 0
            o.append([0.0] * len(v[0]) if v else [])
            lse.append(-math.inf)
            continue
        s = [scale * _dot(q[i], k[j]) for j in keys]
        m = max(s)
        e = [math.exp(x - m) for x in s]
        l = math.fsum(e)
        o.append([math.fsum(e[t] * v[j][d] for t, j in enumerate(keys)) / l for d in range(len(v[0]))])
        lse.append(m + math.log(l))
    return o, lse


def backward(q, k, v, do, causal, scale, window=-1, block_mask=None, block=128):
    """Loop form of dQ, dK, dV for one head (nested lists)."""
    n, dd = len(q), len(q[0])
    nk = len(k)
    p = []
    for i in range(n):
        kept = set(_keys(i, n, nk, causal, window, block_mask, block))
        if not kept:  # a row that keeps no key has P = 0 (its output is the constant 0)
            p.append([0.0] * nk)
            continue
        s = [(scale * _dot(q[i], k[j]) if j in kept else -math.inf) for j in range(nk)]
        m = max(s)
        e = [0.0 if x == -math.inf else math.exp(x - m) for x in s]
        l = math.fsum(e)
        p.append([x / l for x in e])
    dp = [[_dot(do[i], v[j]) for j in range(nk)] for i in range(n)]
    ds = []
    for i in range(n):
        c = math.fsum(p[i][j] * dp[i][j] for j in range(nk))
        ds.append([p[i][j] * (dp[i][j] - c) for j in range(nk)])
    dv = [[math.fsum(p[i][j] * do[i][d] for i in range(n)) for d in range(len(v[0]))] for j in range(nk)]
    dq = [[scale * math.fsum(ds[i][j] * k[j][d] for j in range(nk)) for d in range(dd)] for i in range(n)]
    dk = [[scale * math.fsum(ds[i][j] * q[i][d] for i in range(n)) for d in range(dd)] for j in range(nk)]
    return dq, dk, dv
