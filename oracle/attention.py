"""Exact scaled-dot-product attention in float64 -- oracle (test infrastructure only).

Conventions (the pages fix none of them; these are the plainest readings):
  * tensors are contiguous [B, H, N, D]: queries have N_q rows and keys N_k
    (N_q = N_k unless a call says otherwise);
  * grouped-query attention (named on the page "FlashAttention" entity trail,
    section "Corpus findings", AVO entry): K and V may have Hkv heads with Hkv
    dividing H; query head h then uses K/V head h // (H // Hkv), i.e. each run
    of H // Hkv consecutive query heads shares one K/V head;
  * scores are s_ij = scale * <q_i, k_j>;
  * causal keeps key j only when j <= i + (N_k - N_q): the last query is
    aligned with the last key (bottom-right), as when queries extend a cached
    prefix of keys (the KV-cache prefill named in the FlashPrefill V2 entry of
    the page "FlashAttention" entity trail, section "Corpus findings"); with
    equal lengths this is j <= i;
  * a left window w >= 0 also drops keys j < i + (N_k - N_q) - w, i.e. a row
    keeps at most the w + 1 keys ending at its diagonal (the local
    sliding-window attention of the WAND entry on the "attention mechanism"
    tag page, and the local window of the NanoGPT speedrun post on the "MHA"
    search page); w < 0 means no window;
  * lse_i = log(sum_j exp(s_ij)) with the natural logarithm, over the kept keys;
  * a row that keeps no key (causal with N_k < N_q leaves the first N_q - N_k
    rows so; a packed sequence may have no keys) has an empty sum: lse_i =
    ln 0 = -inf, and its output is taken as 0 (the sum of p_ij v_j over no
    keys), so it does not depend on Q, K or V and its gradients are 0;
  * block sparsity (the customisation the page "FlashAttention (Metal Port)"
    README, section "Documentation", calls easy to add to the base
    algorithm): an optional boolean mask over (query block, key block) pairs
    of ``block`` x ``block`` scores (128 by default) keeps score (i, j) only
    where mask[b, h, i // block, j // block] is true, on top of causal and
    window;
  * packed variable-length batches (``forward_varlen`` / ``backward_varlen``)
    are independent problems, one per sequence: rows cu[b] .. cu[b+1]-1 of the
    packed [total, H, D] tensors are sequence b, with these conventions inside
    each sequence (the continuous batching of the FlashPrefill V2 entry on the
    page "FlashAttention" entity trail, section "Corpus findings").

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


def key_bounds(rows, n_q, n_k, causal, window=-1):
    """First and last key index each query row keeps (inclusive), per the conventions above."""
    rows = np.asarray(rows, dtype=np.int64)
    off = n_k - n_q
    lo = np.maximum(0, rows + off - window) if window >= 0 else np.zeros_like(rows)
    hi = np.minimum(n_k - 1, rows + off) if causal else np.full_like(rows, n_k - 1)
    return lo, hi


def scores(q, k, scale, causal, rows=None, n_q=None, window=-1, block_mask=None, block=128):
    """S[i, j] = scale * q_i . k_j for one head, masked entries set to -inf.

    q: [M, D] (the query rows listed in ``rows``, or all rows 0..M-1), k: [N_k, D];
    n_q: the head's query length (default M); block_mask: this head's boolean
    [ceil(N_q / block), ceil(N_k / block)] block mask, or None.
    """
    q = _as_f64(q)
    k = _as_f64(k)
    s = scale * (q @ k.T)
    idx = np.arange(q.shape[0]) if rows is None else np.asarray(rows)
    n_q = q.shape[0] if n_q is None else n_q
    if causal or window >= 0:
        lo, hi = key_bounds(idx, n_q, k.shape[0], causal, window)
        j = np.arange(k.shape[0])[None, :]
        s = np.where((j < lo[:, None]) | (j > hi[:, None]), -np.inf, s)
    if block_mask is not None:
        bm = np.asarray(block_mask, dtype=bool)
        keep = bm[idx[:, None] // block, np.arange(k.shape[0])[None, :] // block]
        s = np.where(keep, s, -np.inf)
    return s


def softmax_rows(s):
    """Row softmax of a score block; returns (P, lse). Max-subtracted for range only.

    A row whose scores are all -inf keeps no key: its P row is 0 and its lse -inf.
    """
    m = s.max(axis=1) if s.shape[1] else np.full(s.shape[0], -np.inf)
    empty = m == -np.inf
    m0 = np.where(empty, 0.0, m)
    p = np.exp(s - m0[:, None])  # exp(-inf) = 0 on every entry of an empty row
    l = p.sum(axis=1)
    l1 = np.where(empty, 1.0, l)
    lse = np.where(empty, -np.inf, m0 + np.log(l1))
    return p / l1[:, None], lse


def _head_mask(block_mask, b, h):
    return None if block_mask is None else np.asarray(block_mask)[b, h]


def forward(q, k, v, causal, scale, rows=None, window=-1, block_mask=None, block=128):
    """Attention forward for all heads.

    Args:
      q: [B, H, N_q, D]; k, v: [B, Hkv, N_k, D] with Hkv dividing H (any float
        dtype; widened to float64).
      causal: keep key j only for j <= i + N_k - N_q.
      scale: the factor on q.k.
      window: left window (keys j >= i + N_k - N_q - window), < 0 for none.
      rows: optional sorted 1-D array of query indices; when given, only those
        rows are computed (rows are independent, so this is the same result).
      block_mask: optional boolean [B, H, ceil(N_q / block), ceil(N_k / block)]
        mask of kept (query block, key block) pairs.
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
                s = scores(q[b, h, rr], k[b, kh], scale, causal, rows=rr, n_q=N, window=window,
                           block_mask=_head_mask(block_mask, b, h), block=block)
                p, lse_blk = softmax_rows(s)
                o[b, h, r0:r1] = p @ v[b, kh]
                lse[b, h, r0:r1] = lse_blk
    return o, lse


def backward(q, k, v, do, causal, scale, window=-1, block_mask=None, block=128):
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
            s = scores(q[b, h], k[b, kh], scale, causal, window=window, block_mask=_head_mask(block_mask, b, h),
                       block=block)
            p, _ = softmax_rows(s)
            dv[b, kh] += p.T @ do[b, h]
            dp = do[b, h] @ v[b, kh].T
            ds = p * (dp - (p * dp).sum(axis=1, keepdims=True))
            dq[b, h] = scale * (ds @ k[b, kh])
            dk[b, kh] += scale * (ds.T @ q[b, h])
    return dq, dk, dv


def backward_dq_rows(q, k, v, do, causal, scale, rows, window=-1):
    """dQ of the listed query rows only, in float64 (for heads too long to materialise S).

    dQ_i depends on row i alone: with s_i = scale q_i K^T over the kept keys,
    p_i = softmax(s_i), dp_i = dO_i V^T and ds_i = p_i * (dp_i - <p_i, dp_i>),
    dQ_i = scale ds_i K -- the row-i slice of ``backward``'s dQ, the same chain
    rule. rows: sorted 1-D array of query indices. Returns [B, H, len(rows), D].
    """
    q = _as_f64(q)
    k = _as_f64(k)
    v = _as_f64(v)
    do = _as_f64(do)
    B, H, N, D = q.shape
    G = _group(H, k.shape[1])
    sel = np.asarray(rows, dtype=np.int64)
    dq = np.empty((B, H, len(sel), D))
    for b in range(B):
        for h in range(H):
            kh = h // G
            for r0, r1 in _row_blocks(len(sel), k.shape[2]):
                rr = sel[r0:r1]
                s = scores(q[b, h, rr], k[b, kh], scale, causal, rows=rr, n_q=N, window=window)
                p, _ = softmax_rows(s)
                dp = do[b, h, rr] @ v[b, kh].T
                ds = p * (dp - (p * dp).sum(axis=1, keepdims=True))
                dq[b, h, r0:r1] = scale * (ds @ k[b, kh])
    return dq


def backward_kv_rows(q, k, v, do, causal, scale, rows, window=-1):
    """dK and dV of the listed key rows only, in float64 (for heads too long to materialise S).

    Key j's gradients are column j of ``backward``'s chain rule: every query
    row i that keeps key j contributes, through its own probabilities and dP row,
      dS_ij = P_ij * (dP_ij - <P_i, dP_i>),  dK_j = scale sum_i dS_ij q_i,  dV_j = sum_i P_ij dO_i.
    Each such row's P_i and <P_i, dP_i> need all of its kept keys, so the
    scores of those rows are formed in full; only query rows that keep one of
    the listed keys are visited (for causal masking, rows from the first
    listed key's diagonal on). With grouped K/V heads a key's gradients are
    sums over the query heads of its group. rows: sorted 1-D array of key
    indices. Returns (dK, dV), each [B, Hkv, len(rows), D].
    """
    q = _as_f64(q)
    k = _as_f64(k)
    v = _as_f64(v)
    do = _as_f64(do)
    B, H, N, D = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    G = _group(H, Hkv)
    sel = np.asarray(rows, dtype=np.int64)
    dk = np.zeros((B, Hkv, len(sel), D))
    dv = np.zeros((B, Hkv, len(sel), v.shape[-1]))
    if len(sel) == 0:
        return dk, dv
    # query rows that may keep a listed key: lo(i) <= j <= hi(i) for some listed j
    i_all = np.arange(N)
    lo, hi = key_bounds(i_all, N, Nk, causal, window)
    cand = i_all[(hi >= sel.min()) & (lo <= sel.max())]
    for b in range(B):
        for h in range(H):
            kh = h // G
            for r0, r1 in _row_blocks(len(cand), Nk):
                rr = cand[r0:r1]
                s = scores(q[b, h, rr], k[b, kh], scale, causal, rows=rr, n_q=N, window=window)
                p, _ = softmax_rows(s)
                dp = do[b, h, rr] @ v[b, kh].T
                c = (p * dp).sum(axis=1, keepdims=True)
                ps = p[:, sel]
                ds = ps * (dp[:, sel] - c)
                dk[b, kh] += scale * (ds.T @ q[b, h, rr])
                dv[b, kh] += ps.T @ do[b, h, rr]
    return dk, dv


def _check_cu(cu, total, B):
    cu = np.asarray(cu, dtype=np.int64)
    if cu.shape != (B + 1,) or cu[0] != 0 or cu[-1] != total or np.any(np.diff(cu) < 0):
        raise ValueError("cu_seqlens must be [B + 1] non-decreasing offsets from 0 to the packed length")
    return cu


def forward_varlen(q, k, v, cu_q, cu_k, causal, scale, window=-1):
    """Packed variable-length forward: q [T_q, H, D], k, v [T_k, Hkv, D]; sequence b is
    rows cu_q[b] .. cu_q[b+1]-1 of q and cu_k[b] .. cu_k[b+1]-1 of k and v.
    Returns O [T_q, H, D] and lse [H, T_q], float64."""
    q, k, v = _as_f64(q), _as_f64(k), _as_f64(v)
    B = len(cu_q) - 1
    cu_q, cu_k = _check_cu(cu_q, q.shape[0], B), _check_cu(cu_k, k.shape[0], B)
    o = np.zeros((q.shape[0], q.shape[1], v.shape[2]))
    lse = np.full((q.shape[1], q.shape[0]), -np.inf)
    for b in range(B):
        qs, ks = slice(cu_q[b], cu_q[b + 1]), slice(cu_k[b], cu_k[b + 1])
        if cu_q[b + 1] == cu_q[b]:
            continue
        # one sequence as a [1, H, n, D] problem
        ob, lb = forward(q[qs].transpose(1, 0, 2)[None], k[ks].transpose(1, 0, 2)[None],
                         v[ks].transpose(1, 0, 2)[None], causal, scale, window=window)
        o[qs] = ob[0].transpose(1, 0, 2)
        lse[:, qs] = lb[0]
    return o, lse


def backward_varlen(q, k, v, do, cu_q, cu_k, causal, scale, window=-1):
    """Gradients of the packed variable-length forward, one sequence at a time.
    Returns dQ [T_q, H, D], dK and dV [T_k, Hkv, D], float64 (keys of no sequence get 0)."""
    q, k, v, do = _as_f64(q), _as_f64(k), _as_f64(v), _as_f64(do)
    B = len(cu_q) - 1
    cu_q, cu_k = _check_cu(cu_q, q.shape[0], B), _check_cu(cu_k, k.shape[0], B)
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    for b in range(B):
        qs, ks = slice(cu_q[b], cu_q[b + 1]), slice(cu_k[b], cu_k[b + 1])
        t = lambda x, sl: x[sl].transpose(1, 0, 2)[None]
        gq, gk, gv = backward(t(q, qs), t(k, ks), t(v, ks), t(do, qs), causal, scale, window=window)
        dq[qs], dk[ks], dv[ks] = gq[0].transpose(1, 0, 2), gk[0].transpose(1, 0, 2), gv[0].transpose(1, 0, 2)
    return dq, dk, dv
