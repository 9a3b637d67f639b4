"""Plausible mistakes planted in copies of the oracle (on the CPU) must each fail a pin.

This shows the pins are sharp enough to catch a dropped term, a wrong sign,
a wrong index or a transposed operand anywhere in the oracle.
"""
import numpy as np
import pytest

import oracle_pins as pins
from oracle import attention, brute


def _fwd_factory(mask_shift=0, scale_pow=1, use_max=True, lse_log=np.log, transpose_k=False, v_t=False):
    def fwd(q, k, v, causal, scale, rows=None):
        q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
        B, H, N, D = q.shape
        o = np.empty((B, H, N, v.shape[-1]))
        lse = np.empty((B, H, N))
        for b in range(B):
            for h in range(H):
                kk = k[b, h][::-1] if transpose_k else k[b, h]
                s = (scale ** scale_pow) * (q[b, h] @ kk.T)
                if causal:
                    s = np.where(np.arange(N)[None, :] > np.arange(N)[:, None] + mask_shift, -np.inf, s)
                m = s.max(axis=1) if use_max else np.zeros(N)
                p = np.exp(s - m[:, None])
                l = p.sum(axis=1)
                vv = v[b, h][::-1] if v_t else v[b, h]
                o[b, h] = (p @ vv) / l[:, None]
                lse[b, h] = (m if use_max else 0) + lse_log(l)
        return o, lse
    return fwd


FORWARD_MUTANTS = {
    "mask_off_by_one": _fwd_factory(mask_shift=1),
    "mask_excludes_diagonal": _fwd_factory(mask_shift=-1),
    "scale_squared": _fwd_factory(scale_pow=2),
    "lse_log2": _fwd_factory(lse_log=np.log2),
    "keys_reversed": _fwd_factory(transpose_k=True),
    "values_reversed": _fwd_factory(v_t=True),
}


def _all_forward_pins(fwd):
    failures = 0
    for pin in pins.FORWARD_PINS:
        try:
            pin(fwd)
        except AssertionError:
            failures += 1
    try:
        pins.pin_hand_cases(fwd)
    except AssertionError:
        failures += 1
    return failures


def test_unmutated_forward_passes_every_pin():
    assert _all_forward_pins(attention.forward) == 0


@pytest.mark.parametrize("name", sorted(FORWARD_MUTANTS))
def test_forward_mutant_is_caught(name):
    assert _all_forward_pins(FORWARD_MUTANTS[name]) > 0, name


def _bwd_factory(drop_jacobian_term=False, sign=1.0, dk_from_k=False, dv_untransposed=False, no_scale=False):
    def bwd(q, k, v, do, causal, scale):
        q, k, v, do = (np.asarray(x, dtype=np.float64) for x in (q, k, v, do))
        dq, dk, dv = np.empty_like(q), np.empty_like(k), np.empty_like(v)
        B, H, N, D = q.shape
        for b in range(B):
            for h in range(H):
                s = attention.scores(q[b, h], k[b, h], scale, causal)
                p, _ = attention.softmax_rows(s)
                dv[b, h] = (p if dv_untransposed else p.T) @ do[b, h]
                dp = do[b, h] @ v[b, h].T
                c = 0.0 if drop_jacobian_term else (p * dp).sum(axis=1, keepdims=True)
                ds = p * (dp - sign * c)
                f = 1.0 if no_scale else scale
                dq[b, h] = f * (ds @ k[b, h])
                dk[b, h] = f * (ds.T @ (k[b, h] if dk_from_k else q[b, h]))
        return dq, dk, dv
    return bwd


BACKWARD_MUTANTS = {
    "drop_jacobian_term": _bwd_factory(drop_jacobian_term=True),
    "jacobian_sign": _bwd_factory(sign=-1.0),
    "dk_uses_k": _bwd_factory(dk_from_k=True),
    "dv_untransposed": _bwd_factory(dv_untransposed=True),
    "missing_scale": _bwd_factory(no_scale=True),
}


def _all_backward_pins(bwd):
    failures = 0
    for f in (lambda: pins.pin_hand_cases(attention.forward, bwd),
              lambda: pins.pin_backward_identities(bwd),
              lambda: pins.pin_finite_differences(attention.forward, bwd),
              lambda: pins.pin_torch_backward(bwd)):
        try:
            f()
        except AssertionError:
            failures += 1
    return failures


@pytest.mark.parametrize("name", sorted(BACKWARD_MUTANTS))
def test_backward_mutant_is_caught(name):
    assert _all_backward_pins(BACKWARD_MUTANTS[name]) > 0, name


def test_unmutated_backward_passes_every_pin():
    assert _all_backward_pins(attention.backward) == 0


def _gqa_factory(interleaved=False, overwrite=False):
    """A grouped-query forward/backward pair with one planted mistake."""
    def kv_index(h, G, Hkv):
        return h % Hkv if interleaved else h // G

    def fwd(q, k, v, causal, scale, rows=None):
        q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
        B, H, N, D = q.shape
        G = H // k.shape[1]
        o = np.empty((B, H, N, v.shape[-1]))
        lse = np.empty((B, H, N))
        for b in range(B):
            for h in range(H):
                kh = kv_index(h, G, k.shape[1])
                s = attention.scores(q[b, h], k[b, kh], scale, causal)
                p, lse[b, h] = attention.softmax_rows(s)
                o[b, h] = p @ v[b, kh]
        return o, lse

    def bwd(q, k, v, do, causal, scale):
        q, k, v, do = (np.asarray(x, dtype=np.float64) for x in (q, k, v, do))
        B, H, N, D = q.shape
        G = H // k.shape[1]
        dq, dk, dv = np.empty_like(q), np.zeros_like(k), np.zeros_like(v)
        for b in range(B):
            for h in range(H):
                kh = kv_index(h, G, k.shape[1])
                p, _ = attention.softmax_rows(attention.scores(q[b, h], k[b, kh], scale, causal))
                dp = do[b, h] @ v[b, kh].T
                ds = p * (dp - (p * dp).sum(axis=1, keepdims=True))
                dq[b, h] = scale * (ds @ k[b, kh])
                if overwrite:
                    dv[b, kh] = p.T @ do[b, h]
                    dk[b, kh] = scale * (ds.T @ q[b, h])
                else:
                    dv[b, kh] += p.T @ do[b, h]
                    dk[b, kh] += scale * (ds.T @ q[b, h])
        return dq, dk, dv
    return fwd, bwd


@pytest.mark.parametrize("mutant", ["interleaved_heads", "group_grads_overwritten"])
def test_gqa_mutants_fail_a_pin(mutant):
    fwd, bwd = _gqa_factory(interleaved=mutant == "interleaved_heads", overwrite=mutant == "group_grads_overwritten")
    failures = 0
    for pin in (pins.pin_torch_gqa, pins.pin_gqa_matches_copied_heads):
        try:
            pin(fwd, bwd)
        except AssertionError:
            failures += 1
    assert failures >= 1


def test_unmutated_gqa_factory_passes():
    fwd, bwd = _gqa_factory()
    pins.pin_torch_gqa(fwd, bwd)
    pins.pin_gqa_matches_copied_heads(fwd, bwd)


def _mask_factory(top_left=False, window_short=False):
    """The oracle with one planted mistake in the key bounds: top-left causal alignment, or a window one key short."""
    def bounds(rows, n_q, n_k, causal, window):
        rows = np.asarray(rows)
        off = 0 if top_left else n_k - n_q
        w = window - 1 if (window_short and window >= 0) else window
        lo = np.maximum(0, rows + off - w) if window >= 0 else np.zeros_like(rows)
        hi = np.minimum(n_k - 1, rows + off) if causal else np.full_like(rows, n_k - 1)
        return lo, hi

    def head(q, k, causal, scale, window):
        s = scale * (q @ k.T)
        lo, hi = bounds(np.arange(q.shape[0]), q.shape[0], k.shape[0], causal, window)
        j = np.arange(k.shape[0])[None, :]
        return np.where((j < lo[:, None]) | (j > hi[:, None]), -np.inf, s)

    def fwd(q, k, v, causal, scale, rows=None, window=-1):
        q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
        B, H, N, _ = q.shape
        o, lse = np.empty((B, H, N, v.shape[-1])), np.empty((B, H, N))
        for b in range(B):
            for h in range(H):
                p, lse[b, h] = attention.softmax_rows(head(q[b, h], k[b, h], causal, scale, window))
                o[b, h] = p @ v[b, h]
        return o, lse

    def bwd(q, k, v, do, causal, scale, window=-1):
        q, k, v, do = (np.asarray(x, dtype=np.float64) for x in (q, k, v, do))
        dq, dk, dv = np.empty_like(q), np.empty_like(k), np.empty_like(v)
        B, H = q.shape[:2]
        for b in range(B):
            for h in range(H):
                p, _ = attention.softmax_rows(head(q[b, h], k[b, h], causal, scale, window))
                dv[b, h] = p.T @ do[b, h]
                dp = do[b, h] @ v[b, h].T
                ds = p * (dp - (p * dp).sum(axis=1, keepdims=True))
                dq[b, h] = scale * (ds @ k[b, h])
                dk[b, h] = scale * (ds.T @ q[b, h])
        return dq, dk, dv
    return fwd, bwd


@pytest.mark.parametrize("mutant", ["top_left_causal", "window_one_short"])
def test_mask_mutants_fail_a_pin(mutant):
    fwd, bwd = _mask_factory(top_left=mutant == "top_left_causal", window_short=mutant == "window_one_short")
    checks = [lambda: pins.pin_torch_lower_right(fwd, bwd), lambda: pins.pin_window_closed_forms(fwd),
              lambda: pins.pin_window_equals_key_slice(fwd), lambda: pins.pin_brute_force_masks(fwd, bwd, brute)]
    failures = 0
    for c in checks:
        try:
            c()
        except (AssertionError, ValueError):
            failures += 1
    assert failures >= 1


def test_unmutated_mask_factory_passes():
    fwd, bwd = _mask_factory()
    pins.pin_torch_lower_right(fwd, bwd)
    pins.pin_window_closed_forms(fwd)
    pins.pin_window_equals_key_slice(fwd)
    pins.pin_brute_force_masks(fwd, bwd, brute)


def _empty_factory(nan_rows=False, lse_zero=False):
    """The oracle with one planted mistake in rows that keep no key: the plain softmax (0/0 there),
    or lse = 0 instead of -inf for them."""
    def softmax(s):
        if nan_rows:
            with np.errstate(invalid="ignore", divide="ignore"):
                m = s.max(axis=1)
                p = np.exp(s - m[:, None])
                l = p.sum(axis=1)
                return p / l[:, None], m + np.log(l)
        p, lse = attention.softmax_rows(s)
        return p, (np.where(lse == -np.inf, 0.0, lse) if lse_zero else lse)

    def fwd(q, k, v, causal, scale, rows=None, window=-1):
        q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
        B, H, N, _ = q.shape
        o, lse = np.empty((B, H, N, v.shape[-1])), np.empty((B, H, N))
        for b in range(B):
            for h in range(H):
                p, lse[b, h] = softmax(attention.scores(q[b, h], k[b, h], scale, causal, window=window))
                o[b, h] = p @ v[b, h]
        return o, lse

    def bwd(q, k, v, do, causal, scale, window=-1):
        q, k, v, do = (np.asarray(x, dtype=np.float64) for x in (q, k, v, do))
        dq, dk, dv = np.empty_like(q), np.empty_like(k), np.empty_like(v)
        B, H = q.shape[:2]
        for b in range(B):
            for h in range(H):
                p, _ = softmax(attention.scores(q[b, h], k[b, h], scale, causal, window=window))
                dv[b, h] = p.T @ do[b, h]
                dp = do[b, h] @ v[b, h].T
                ds = p * (dp - (p * dp).sum(axis=1, keepdims=True))
                dq[b, h] = scale * (ds @ k[b, h])
                dk[b, h] = scale * (ds.T @ q[b, h])
        return dq, dk, dv
    return fwd, bwd


@pytest.mark.parametrize("mutant", ["nan_rows", "lse_zero"])
def test_empty_row_mutants_fail_a_pin(mutant):
    fwd, bwd = _empty_factory(nan_rows=mutant == "nan_rows", lse_zero=mutant == "lse_zero")
    with pytest.raises((AssertionError, ValueError)):
        pins.pin_empty_rows(fwd, bwd)


def test_unmutated_empty_factory_passes():
    pins.pin_empty_rows(*_empty_factory())


def _varlen_factory(key_overrun=False, global_diagonal=False):
    """Packed sequences through the oracle's per-head forward and backward with one planted
    mistake: each sequence also sees the next sequence's first key, or the causal diagonal of every
    sequence is placed from the longest lengths instead of its own."""
    def run(q, k, v, do, cu_q, cu_k, causal, scale, window):
        B = len(cu_q) - 1
        nq, nk = np.diff(cu_q), np.diff(cu_k)
        Lq, Lk = nq.max(), nk.max()
        o, lse = np.zeros((q.shape[0], q.shape[1], v.shape[2])), np.full((q.shape[1], q.shape[0]), -np.inf)
        dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
        G = q.shape[1] // k.shape[1]
        for b in range(B):
            qs = slice(cu_q[b], cu_q[b + 1])
            ks = slice(cu_k[b], min(cu_k[b + 1] + (1 if key_overrun else 0), k.shape[0]))
            n_q = nk[b] - (Lk - Lq) if global_diagonal else nq[b]
            for h in range(q.shape[1]):
                qh, kh, vh = q[qs, h], k[ks, h // G], v[ks, h // G]
                s = attention.scores(qh, kh, scale, causal, rows=np.arange(nq[b]), n_q=n_q, window=window)
                p, l = attention.softmax_rows(s)
                o[qs, h], lse[h, qs] = p @ vh, l
                dp = do[qs, h] @ vh.T
                ds = p * (dp - (p * dp).sum(axis=1, keepdims=True))
                dq[qs, h] = scale * (ds @ kh)
                dk[ks, h // G] += scale * (ds.T @ qh)
                dv[ks, h // G] += p.T @ do[qs, h]
        return (o, lse), (dq, dk, dv)

    def fwd(q, k, v, cu_q, cu_k, causal, scale, window=-1):
        return run(q, k, v, np.zeros_like(q), cu_q, cu_k, causal, scale, window)[0]

    def bwd(q, k, v, do, cu_q, cu_k, causal, scale, window=-1):
        return run(q, k, v, do, cu_q, cu_k, causal, scale, window)[1]
    return fwd, bwd


@pytest.mark.parametrize("mutant", ["key_overrun", "global_diagonal"])
def test_varlen_mutants_fail_a_pin(mutant):
    fwd, bwd = _varlen_factory(key_overrun=mutant == "key_overrun", global_diagonal=mutant == "global_diagonal")
    with pytest.raises((AssertionError, ValueError)):
        pins.pin_varlen_padded(fwd, bwd)


def test_unmutated_varlen_factory_passes():
    pins.pin_varlen_padded(*_varlen_factory())


def _block_factory(mutant=None):
    """The oracle with one planted mistake in the block-mask lookup: the query block taken one row
    late, or the key block index replaced by the query's."""
    def head_scores(qh, kh, scale, causal, window, bm, block, n_q):
        s = attention.scores(qh, kh, scale, causal, window=window, n_q=n_q)
        if bm is None:
            return s
        i = np.arange(qh.shape[0])[:, None]
        j = np.arange(kh.shape[0])[None, :]
        if mutant == "row_late":
            ib = np.minimum((i + 1) // block, bm.shape[0] - 1)
            keep = bm[ib, j // block]
        elif mutant == "key_from_query":
            keep = bm[i // block, np.minimum(i // block, bm.shape[1] - 1)] & np.ones_like(j, dtype=bool)
        else:
            keep = bm[i // block, j // block]
        return np.where(keep, s, -np.inf)

    def fwd(q, k, v, causal, scale, rows=None, window=-1, block_mask=None, block=128):
        q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
        B, H, N, _ = q.shape
        G = H // k.shape[1]
        o, lse = np.empty((B, H, N, v.shape[-1])), np.empty((B, H, N))
        for b in range(B):
            for h in range(H):
                bm = None if block_mask is None else np.asarray(block_mask)[b, h]
                p, lse[b, h] = attention.softmax_rows(head_scores(q[b, h], k[b, h // G], scale, causal, window, bm,
                                                                  block, N))
                o[b, h] = p @ v[b, h // G]
        return o, lse

    def bwd(q, k, v, do, causal, scale, window=-1, block_mask=None, block=128):
        q, k, v, do = (np.asarray(x, dtype=np.float64) for x in (q, k, v, do))
        dq, dk, dv = np.empty_like(q), np.zeros_like(k), np.zeros_like(v)
        B, H, N, _ = q.shape
        G = H // k.shape[1]
        for b in range(B):
            for h in range(H):
                bm = None if block_mask is None else np.asarray(block_mask)[b, h]
                kh, vh = k[b, h // G], v[b, h // G]
                p, _ = attention.softmax_rows(head_scores(q[b, h], kh, scale, causal, window, bm, block, N))
                dv[b, h // G] += p.T @ do[b, h]
                dp = do[b, h] @ vh.T
                ds = p * (dp - (p * dp).sum(axis=1, keepdims=True))
                dq[b, h] = scale * (ds @ kh)
                dk[b, h // G] += scale * (ds.T @ q[b, h])
        return dq, dk, dv
    return fwd, bwd


@pytest.mark.parametrize("mutant", ["row_late", "key_from_query"])
def test_block_mask_mutants_fail_a_pin(mutant):
    fwd, bwd = _block_factory(mutant)
    failures = 0
    for c in (lambda: pins.pin_block_mask_torch(fwd, bwd), lambda: pins.pin_block_mask_drops_keys(fwd),
              lambda: pins.pin_block_mask_brute(fwd, bwd, brute)):
        try:
            c()
        except (AssertionError, ValueError, IndexError):
            failures += 1
    assert failures >= 1


def test_unmutated_block_factory_passes():
    fwd, bwd = _block_factory()
    pins.pin_block_mask_all_true(fwd, bwd)
    pins.pin_block_mask_torch(fwd, bwd)
    pins.pin_block_mask_drops_keys(fwd)
    pins.pin_block_mask_brute(fwd, bwd, brute)


def _dq_rows_factory(mutant=None):
    """Copies of the row-sampled dQ with one planted mistake each."""

    def dq_rows(q, k, v, do, causal, scale, rows, window=-1):
        q, k, v, do = (np.asarray(x, dtype=np.float64) for x in (q, k, v, do))
        B, H, N, D = q.shape
        G = H // k.shape[1]
        rows = np.asarray(rows)
        src = np.minimum(rows + 1, N - 1) if mutant == "row_shift" else rows
        out = np.empty((B, H, len(rows), D))
        for b in range(B):
            for h in range(H):
                kk, vv = k[b, h // G], v[b, h // G]
                n_q = N if mutant != "top_left" else kk.shape[0]
                s = attention.scores(q[b, h, src], kk, scale, causal, rows=src, n_q=n_q, window=window)
                p, _ = attention.softmax_rows(s)
                dp = do[b, h, src] @ vv.T
                c = 0.0 if mutant == "no_jacobian" else (p * dp).sum(axis=1, keepdims=True)
                ds = p * (dp - c)
                out[b, h] = (1.0 if mutant == "no_scale" else scale) * (ds @ kk)
        return out

    return dq_rows


@pytest.mark.parametrize("mutant", ["row_shift", "top_left", "no_jacobian", "no_scale"])
def test_dq_rows_mutants_fail_a_pin(mutant):
    f = _dq_rows_factory(mutant)
    failures = 0
    for pin in (lambda: pins.pin_dq_rows_brute(f, brute), lambda: pins.pin_dq_rows_torch(f)):
        try:
            pin()
        except AssertionError:
            failures += 1
    assert failures > 0, mutant


def test_unmutated_dq_rows_factory_passes():
    f = _dq_rows_factory()
    pins.pin_dq_rows_brute(f, brute)
    pins.pin_dq_rows_torch(f)


def _kv_rows_factory(mutant=None):
    """Copies of the row-sampled dK / dV with one planted mistake each."""

    def kv_rows(q, k, v, do, causal, scale, rows, window=-1):
        q, k, v, do = (np.asarray(x, dtype=np.float64) for x in (q, k, v, do))
        B, H, N, D = q.shape
        G = H // k.shape[1]
        rows = np.asarray(rows)
        cols = np.minimum(rows + 1, k.shape[2] - 1) if mutant == "row_shift" else rows
        dk = np.zeros((B, k.shape[1], len(rows), D))
        dv = np.zeros_like(dk)
        # the "late_queries" mutant visits only query rows from the last listed key on
        first = int(rows.max()) - (k.shape[2] - N) if mutant == "late_queries" else 0
        qr = np.arange(max(0, first), N)
        for b in range(B):
            for h in range(H):
                kk, vv = k[b, h // G], v[b, h // G]
                s = attention.scores(q[b, h, qr], kk, scale, causal, rows=qr, n_q=N, window=window)
                p, _ = attention.softmax_rows(s)
                dp = do[b, h, qr] @ vv.T
                c = 0.0 if mutant == "no_jacobian" else (p * dp).sum(axis=1, keepdims=True)
                ds = p[:, cols] * (dp[:, cols] - c)
                sc = 1.0 if mutant == "no_scale" else scale
                kh = h // G
                if mutant == "overwrite" and h % G:
                    dk[b, kh] = 0.0
                    dv[b, kh] = 0.0
                dk[b, kh] += sc * (ds.T @ q[b, h, qr])
                dv[b, kh] += (dp[:, cols] if mutant == "dp_for_p" else p[:, cols]).T @ do[b, h, qr]
        return dk, dv

    return kv_rows


@pytest.mark.parametrize("mutant", ["row_shift", "late_queries", "no_jacobian", "no_scale", "overwrite",
                                    "dp_for_p"])
def test_kv_rows_mutants_fail_a_pin(mutant):
    f = _kv_rows_factory(mutant)
    failures = 0
    for pin in (lambda: pins.pin_kv_rows_brute(f, brute), lambda: pins.pin_kv_rows_torch(f)):
        try:
            pin()
        except AssertionError:
            failures += 1
    assert failures > 0, mutant


def test_unmutated_kv_rows_factory_passes():
    f = _kv_rows_factory()
    pins.pin_kv_rows_brute(f, brute)
    pins.pin_kv_rows_torch(f)
