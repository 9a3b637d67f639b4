"""Exact scaled-dot-product attention in float64 -- oracle (test infrastructure only).

Conventions (the pages fix none of them; these are the plainest readings):
  * tensors are contiguous [B, H, N, D]; queries and keys have the same length N;
  * grouped-query attention (named on the page "FlashAttention" entity trail,
    section "Corpus findings", AVO entry): K and V may have Hkv heads with Hkv
    dividing H; query head h then uses K/V head h // (H // Hkv), i.e. each run
    of H // Hkv consecutive query heads shares one K/V head;
  * scores are s_ij = scale * <q_i, k_j>;
  * causal keeps key j only when j <= i (with equal query and key lengths the
    top-left and bottom-right alignments coincide, and no row is empty);
  * lse_i = log(sum_j exp(s_ij)) with the natural logarithm, over the kept keys.

The method on the pages (tiling, online softmax, deferred normalisation,
conditional rescaling -- page "r/mlscaling", FA1-FA4 version list) reaches this
result exactly up to rounding, so the oracle is the definition itself with the
N x N score matrix materialised. Rows of a head are independent by definition;
long heads are processed a block of rows at a time only to bound memory.
"""
from __future__ import annotations

import numpy as np

_ROW_BLOCK_BYTES = 1 << 28  # bound on one materialised block of S (256 MiB)


def _as_f64(x):
    return np.asarray(x, dtype=np.float64)


def _row_blocks(n_rows, n_cols):
    rows = max(1, _ROW_BLOCK_BYTES // (8 * max(1, n_cols)))
    for r0 in range(0, n_rows, rows):
        yield r0, min(n_rows, r0 + rows)


def _group(h_q, h_kv):
    """Query heads per K/V head; H_kv must divide H_q."""
    if h_kv < 1 or h_q % h_kv:
        raise ValueError(f"K/V heads ({h_kv}) must divide query heads ({h_q})")
    return h_q // h_kv


def scores(q, k, scale, causal, rows=None):
    """S[i, j] = scale * q_i . k_j for one head, masked entries set to -inf.

    q: [M, D] (the query rows listed in ``rows``, or all rows 0..M-1), k: [N, D].
    """
    q = _as_f64(q)
    k = _as_f64(k)
    s = scale * (q @ k.T)
    if causal:
        idx = np.arange(q.shape[0]) if rows is None else np.asarray(rows)
        s = np.where(np.arange(k.shape[0])[None, :] > idx[:, None], -np.inf, s)
    return s


def softmax_rows(s):
    """Row softmax of a score block; returns (P, lse). Max-subtracted for range only."""
    m = s.max(axis=1)
    p = np.exp(s - m[:, None])
    l = p.sum(axis=1)
    return p / l[:, None], m + np.log(l)


def forward(q, k, v, causal, scale, rows=None):
    """Attention forward for all heads.

    Args:
      q: [B, H, N, D]; k, v: [B, Hkv, N, D] with Hkv dividing H (any float
        dtype; widened to float64).
      causal: keep key j only for j <= i.
      scale: the factor on q.k.
      rows: optional sorted 1-D array of query indices; when given, only those
        rows are computed (rows are independent, so this is the same result).
    Returns:
      O  [B, H, M, D] float64 and lse [B, H, M] float64 (M = N or len(rows)).
    """
    q = _as_f64(q)
    k = _as_f64(k)
    v = _as_f64(v)
    B, H, N, D = q.shape
    G = _group(H, k.shape[1])
    sel = np.arange(N) if rows is None else np.asarray(rows, dtype=np.int64)
    M = sel.shape[0]
    o = np.empty((B, H, M, v.shape[-1]))
    lse = np.empty((B, H, M))
    for b in range(B):
        for h in range(H):
            kh = h // G
            for r0, r1 in _row_blocks(M, k.shape[2]):
                rr = sel[r0:r1]
                s = scores(q[b, h, rr], k[b, kh], scale, causal, rows=rr)
                p, lse_blk = softmax_rows(s)
                o[b, h, r0:r1] = p @ v[b, kh]
                lse[b, h, r0:r1] = lse_blk
    return o, lse


def backward(q, k, v, do, causal, scale):
    """Gradients of sum(dO * O) with respect to Q, K and V, in float64.

    Follows the chain rule through the definition O = softmax(S) V with
    S = scale Q K^T:
      dV = P^T dO
      dP = dO V^T
      dS_i = P_i * (dP_i - <P_i, dP_i>)      (row-wise softmax Jacobian)
      dQ = scale dS K,   dK = scale dS^T Q
    With grouped K/V heads (k, v of shape [B, Hkv, N, D]) a K/V head's dK and
    dV are sums over the query heads that use it, as the chain rule gives for
    a shared input.
    Returns (dQ, dK, dV): dQ [B, H, N, D], dK and dV shaped like k and v, float64.
    """
    q = _as_f64(q)
    k = _as_f64(k)
    v = _as_f64(v)
    do = _as_f64(do)
    dq = np.empty_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    B, H, N, D = q.shape
    G = _group(H, k.shape[1])
    for b in range(B):
        for h in range(H):
            kh = h // G
            s = scores(q[b, h], k[b, kh], scale, causal)
            p, _ = softmax_rows(s)
            dv[b, kh] += p.T @ do[b, h]
            dp = do[b, h] @ v[b, kh].T
            ds = p * (dp - (p * dp).sum(axis=1, keepdims=True))
            dq[b, h] = scale * (ds @ k[b, kh])
            dk[b, kh] += scale * (ds.T @ q[b, h])
    return dq, dk, dv
