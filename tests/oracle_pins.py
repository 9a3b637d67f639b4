"""Checks that pin the oracle to facts other than itself.

Each ``pin_*`` function takes the forward and/or backward implementation to
check (``oracle.attention.forward`` / ``backward`` normally; a deliberately
broken copy in ``test_oracle_mutations.py``) and raises AssertionError when
the implementation disagrees with the fact it encodes. The facts come from
the definition of softmax attention and from calculus, not from the oracle's
own code:

  * hand-derived worked examples (tests/golden/hand_cases.json);
  * closed forms: Q = 0 gives the (prefix) mean of V with lse = ln(count);
    equal key rows give constant scores, lse = c + ln N and O = mean(V);
    V = 1 gives O = 1 (softmax rows sum to one);
  * invariances: a shared permutation of K and V rows (non-causal), adding
    the same vector to every key row (shifts lse by scale*q.u, leaves O),
    rescaling q by c and scale by 1/c;
  * torch's CPU float64 scaled_dot_product_attention and autograd of the
    plain formula (library routines);
  * central finite differences of the forward for the backward;
  * exact backward identities: sum_j dK_j = 0, sum_j dV_j = sum_i dO_i, and
    dQ = dK = 0 when all value rows are equal;
  * query and key lengths that differ, with the causal diagonal aligned at
    the bottom right: torch's causal_lower_right attention bias and autograd;
  * left windows: closed forms (a zero window keeps exactly the diagonal key;
    a window covering every key changes nothing) and, row by row, plain
    attention over the slice of keys the window keeps;
  * grouped K/V heads: torch's scaled_dot_product_attention with enable_gqa
    and its autograd, and the identity that a group's shared K/V head gives
    the same outputs as every query head holding its own copy (whose dK and dV
    then add up to the shared head's);
  * rows that keep no key (causal with fewer keys than queries, no keys at
    all): O = 0 and lse = -inf exactly, the other rows equal torch's
    top-left causal attention of the remaining queries, with zero gradients
    for the empty rows and torch autograd for the rest;
  * block-sparse masks: an all-true mask changes nothing; torch's
    scaled_dot_product_attention and autograd with the element mask expanded
    from the block mask (np.kron) and intersected with the causal / window
    band; masking out whole key blocks equals deleting those keys; and the
    scalar-loop brute force with a block mask;
  * packed variable-length batches: torch's scaled_dot_product_attention and
    autograd on the zero-padded batch with an explicit boolean mask built from
    the lengths (a formulation by masking, not by slicing), including empty
    sequences on either side.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_cases.json")

_SYMBOLS = {"ln2": math.log(2.0), "ln3": math.log(3.0), "ln4": math.log(4.0)}


def _val(x):
    if isinstance(x, str):
        return float(eval(x, {"__builtins__": {}}, dict(_SYMBOLS)))  # symbols only
    return float(x)


def _arr(rows):
    return np.array([[_val(x) for x in r] for r in rows], dtype=np.float64)


def load_hand_cases():
    with open(GOLDEN) as f:
        return json.load(f)["cases"]


def _rand(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


def pin_hand_cases(fwd, bwd=None, tol=1e-12):
    for c in load_hand_cases():
        q, k, v = (_arr(c[n])[None, None] for n in ("q", "k", "v"))
        o, lse = fwd(q, k, v, c["causal"], c["scale"])
        np.testing.assert_allclose(o[0, 0], _arr(c["o"]), atol=tol, err_msg=c["name"])
        np.testing.assert_allclose(lse[0, 0], [_val(x) for x in c["lse"]], atol=tol, err_msg=c["name"])
        if bwd is not None and "do" in c:
            do = _arr(c["do"])[None, None]
            dq, dk, dv = bwd(q, k, v, do, c["causal"], c["scale"])
            for name, got in (("dq", dq), ("dk", dk), ("dv", dv)):
                np.testing.assert_allclose(got[0, 0], _arr(c[name]), atol=tol, err_msg=c["name"] + name)


def pin_zero_query(fwd, N=37, D=8, tol=1e-12):
    """Q = 0: every kept score is 0, so weights are uniform over the kept keys."""
    v = _rand((2, 3, N, D), 1)
    k = _rand((2, 3, N, D), 2)
    q = np.zeros((2, 3, N, D))
    o, lse = fwd(q, k, v, False, 0.3)
    np.testing.assert_allclose(o, np.broadcast_to(v.mean(axis=2, keepdims=True), o.shape), atol=tol)
    np.testing.assert_allclose(lse, math.log(N), atol=tol)
    o, lse = fwd(q, k, v, True, 0.3)
    counts = np.arange(1, N + 1, dtype=np.float64)
    prefix_mean = np.cumsum(v, axis=2) / counts[None, None, :, None]
    np.testing.assert_allclose(o, prefix_mean, atol=tol)
    np.testing.assert_allclose(lse, np.broadcast_to(np.log(counts), lse.shape), atol=tol)


def pin_constant_scores(fwd, N=29, D=16, tol=1e-11):
    """All key rows equal to u: s_ij = scale q_i.u for every j."""
    q = _rand((1, 2, N, D), 3)
    u = _rand((D,), 4)
    k = np.broadcast_to(u, (1, 2, N, D)).copy()
    v = _rand((1, 2, N, D), 5)
    scale = 0.7
    o, lse = fwd(q, k, v, False, scale)
    c = scale * (q @ u)
    np.testing.assert_allclose(lse, c + math.log(N), atol=tol)
    np.testing.assert_allclose(o, np.broadcast_to(v.mean(axis=2, keepdims=True), o.shape), atol=tol)


def pin_ones_value(fwd, N=23, D=4, tol=1e-12):
    """V = 1: softmax rows sum to one, so every output entry is exactly 1."""
    q, k = _rand((1, 1, N, D), 6, 3.0), _rand((1, 1, N, D), 7, 3.0)
    for causal in (False, True):
        o, _ = fwd(q, k, np.ones((1, 1, N, D)), causal, 1.0)
        np.testing.assert_allclose(o, 1.0, atol=tol)


def pin_permutation(fwd, N=41, D=8, tol=1e-12):
    """The non-causal result does not depend on the order of the (key, value) pairs."""
    q, k, v = _rand((1, 2, N, D), 8), _rand((1, 2, N, D), 9), _rand((1, 2, N, 5), 10)
    perm = np.random.default_rng(11).permutation(N)
    o1, l1 = fwd(q, k, v, False, 0.4)
    o2, l2 = fwd(q, k[:, :, perm], v[:, :, perm], False, 0.4)
    np.testing.assert_allclose(o1, o2, atol=tol)
    np.testing.assert_allclose(l1, l2, atol=tol)


def pin_key_shift(fwd, N=33, D=8, tol=1e-11):
    """k_j -> k_j + u adds scale q_i.u to every score of row i: O unchanged, lse shifted."""
    q, k, v = _rand((1, 2, N, D), 12), _rand((1, 2, N, D), 13), _rand((1, 2, N, D), 14)
    u = _rand((D,), 15, 2.0)
    scale = 0.6
    for causal in (False, True):
        o1, l1 = fwd(q, k, v, causal, scale)
        o2, l2 = fwd(q, k + u, v, causal, scale)
        np.testing.assert_allclose(o2, o1, atol=tol)
        np.testing.assert_allclose(l2, l1 + scale * (q @ u), atol=tol)


def pin_scale_fold(fwd, N=19, D=8, tol=1e-12):
    """(c q) and scale / c give the same scores as q and scale."""
    q, k, v = _rand((1, 1, N, D), 16), _rand((1, 1, N, D), 17), _rand((1, 1, N, D), 18)
    for causal in (False, True):
        o1, l1 = fwd(q, k, v, causal, 0.5)
        o2, l2 = fwd(2.5 * q, k, v, causal, 0.2)
        np.testing.assert_allclose(o1, o2, atol=tol)
        np.testing.assert_allclose(l1, l2, atol=tol)


def pin_torch_forward(fwd, tol=1e-12):
    """torch CPU float64 scaled_dot_product_attention (a library routine) on small shapes."""
    import torch

    for (B, H, N, D, causal, seed) in [(2, 3, 17, 8, False, 20), (1, 2, 31, 16, True, 21), (1, 1, 5, 64, True, 22)]:
        q, k, v = (_rand((B, H, N, D), seed + i) for i in range(3))
        scale = 1.0 / math.sqrt(D) * 1.3
        o, lse = fwd(q, k, v, causal, scale)
        tq, tk, tv = (torch.from_numpy(x) for x in (q, k, v))
        ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=causal, scale=scale)
        np.testing.assert_allclose(o, ref.numpy(), atol=tol)
        s = scale * (tq @ tk.transpose(-1, -2))
        if causal:
            s = s.masked_fill(torch.ones(N, N, dtype=torch.bool).triu(1), float("-inf"))
        np.testing.assert_allclose(lse, torch.logsumexp(s, dim=-1).numpy(), atol=tol)


def pin_torch_backward(bwd, tol=1e-11):
    """Autograd (torch CPU float64) of the plain formula sum(dO * softmax(scale QK^T + mask) V)."""
    import torch

    for (B, H, N, D, causal, seed) in [(1, 2, 13, 8, False, 30), (2, 1, 24, 16, True, 31)]:
        q, k, v, do = (_rand((B, H, N, D), seed + i) for i in range(4))
        scale = 0.37
        dq, dk, dv = bwd(q, k, v, do, causal, scale)
        tq, tk, tv = (torch.from_numpy(x).requires_grad_(True) for x in (q, k, v))
        s = scale * (tq @ tk.transpose(-1, -2))
        if causal:
            s = s.masked_fill(torch.ones(N, N, dtype=torch.bool).triu(1), float("-inf"))
        o = torch.softmax(s, dim=-1) @ tv
        (o * torch.from_numpy(do)).sum().backward()
        for got, t in ((dq, tq), (dk, tk), (dv, tv)):
            np.testing.assert_allclose(got, t.grad.numpy(), atol=tol)


def pin_finite_differences(fwd, bwd, tol=1e-7):
    """Central differences of L = sum(dO * O) against the analytic gradients (N, D <= 8)."""
    for (N, D, causal, seed) in [(6, 4, False, 40), (8, 3, True, 41)]:
        q, k, v, do = (_rand((1, 1, N, D), seed + i) for i in range(4))
        scale = 0.8
        dq, dk, dv = bwd(q, k, v, do, causal, scale)
        h = 1e-5

        def loss(q_, k_, v_):
            return float((fwd(q_, k_, v_, causal, scale)[0] * do).sum())

        for which, grad in ((0, dq), (1, dk), (2, dv)):
            fd = np.zeros_like(grad)
            for idx in np.ndindex(*q.shape):
                args = [q.copy(), k.copy(), v.copy()]
                args[which][idx] += h
                lp = loss(*args)
                args[which][idx] -= 2 * h
                lm = loss(*args)
                fd[idx] = (lp - lm) / (2 * h)
            np.testing.assert_allclose(grad, fd, atol=tol)


def pin_backward_identities(bwd, N=45, D=8, tol=1e-12):
    """Identities of the exact gradient, for any inputs."""
    q, k, v, do = (_rand((1, 2, N, D), 50 + i) for i in range(4))
    for causal in (False, True):
        dq, dk, dv = bwd(q, k, v, do, causal, 0.45)
        # rows of dS sum to zero => sum_j dK_j = scale * sum_i (sum_j dS_ij) q_i = 0
        np.testing.assert_allclose(dk.sum(axis=2), 0.0, atol=tol)
        # rows of P sum to one => sum_j dV_j = sum_i dO_i
        np.testing.assert_allclose(dv.sum(axis=2), do.sum(axis=2), atol=tol)
    # all value rows equal => O is constant in Q and K => dQ = dK = 0
    v_eq = np.broadcast_to(_rand((D,), 60), q.shape).copy()
    for causal in (False, True):
        dq, dk, _ = bwd(q, k, v_eq, do, causal, 0.45)
        np.testing.assert_allclose(dq, 0.0, atol=tol)
        np.testing.assert_allclose(dk, 0.0, atol=tol)


def pin_brute_force(fwd, bwd, brute, tol=1e-12):
    """Pure-Python loops (math.fsum / math.exp) on N <= 16."""
    for (N, D, causal, seed) in [(1, 3, False, 70), (7, 5, True, 71), (16, 8, False, 72), (16, 4, True, 73)]:
        q, k, v, do = (_rand((1, 1, N, D), seed + i) for i in range(4))
        scale = 0.9
        o, lse = fwd(q, k, v, causal, scale)
        bo, blse = brute.forward(q[0, 0].tolist(), k[0, 0].tolist(), v[0, 0].tolist(), causal, scale)
        np.testing.assert_allclose(o[0, 0], np.array(bo), atol=tol)
        np.testing.assert_allclose(lse[0, 0], np.array(blse), atol=tol)
        if bwd is not None:
            g = bwd(q, k, v, do, causal, scale)
            bg = brute.backward(q[0, 0].tolist(), k[0, 0].tolist(), v[0, 0].tolist(), do[0, 0].tolist(), causal, scale)
            for got, ref in zip(g, bg):
                np.testing.assert_allclose(got[0, 0], np.array(ref), atol=tol)


def pin_torch_gqa(fwd, bwd, tol=1e-11):
    """torch CPU float64 scaled_dot_product_attention(enable_gqa=True) and its autograd (library routines)."""
    import torch

    for (B, H, Hkv, N, D, causal, seed) in [(2, 6, 2, 19, 8, False, 60), (1, 4, 1, 23, 16, True, 61),
                                             (1, 8, 4, 9, 8, True, 62)]:
        q, do = _rand((B, H, N, D), seed), _rand((B, H, N, D), seed + 3)
        k, v = _rand((B, Hkv, N, D), seed + 1), _rand((B, Hkv, N, D), seed + 2)
        scale = 1.0 / math.sqrt(D) * 0.9
        o, lse = fwd(q, k, v, causal, scale)
        tq, tk, tv = (torch.from_numpy(x).requires_grad_() for x in (q, k, v))
        ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=causal, scale=scale,
                                                               enable_gqa=True)
        np.testing.assert_allclose(o, ref.detach().numpy(), atol=tol)
        ref.backward(torch.from_numpy(do))
        dq, dk, dv = bwd(q, k, v, do, causal, scale)
        assert dk.shape == k.shape and dv.shape == v.shape
        for mine, theirs in ((dq, tq), (dk, tk), (dv, tv)):
            np.testing.assert_allclose(mine, theirs.grad.numpy(), atol=tol)


def pin_gqa_matches_copied_heads(fwd, bwd, tol=1e-12):
    """Sharing a K/V head across a group equals giving each query head its own copy; shared grads are sums."""
    B, H, Hkv, N, D = 2, 6, 3, 17, 8
    G = H // Hkv
    for causal in (False, True):
        q, do = _rand((B, H, N, D), 70), _rand((B, H, N, D), 73)
        k, v = _rand((B, Hkv, N, D), 71), _rand((B, Hkv, N, D), 72)
        kr, vr = np.repeat(k, G, axis=1), np.repeat(v, G, axis=1)  # query head h gets copy of K/V head h // G
        o, lse = fwd(q, k, v, causal, 0.4)
        o_r, lse_r = fwd(q, kr, vr, causal, 0.4)
        np.testing.assert_allclose(o, o_r, atol=tol)
        np.testing.assert_allclose(lse, lse_r, atol=tol)
        dq, dk, dv = bwd(q, k, v, do, causal, 0.4)
        dq_r, dk_r, dv_r = bwd(q, kr, vr, do, causal, 0.4)
        np.testing.assert_allclose(dq, dq_r, atol=tol)
        np.testing.assert_allclose(dk, dk_r.reshape(B, Hkv, G, N, D).sum(axis=2), atol=tol)
        np.testing.assert_allclose(dv, dv_r.reshape(B, Hkv, G, N, D).sum(axis=2), atol=tol)


def pin_torch_lower_right(fwd, bwd, tol=1e-11):
    """torch CPU float64 sdpa with the causal_lower_right bias (a library routine), N_q != N_k, and its autograd."""
    import torch
    from torch.nn.attention.bias import causal_lower_right

    for (B, H, Nq, Nk, D, causal, seed) in [(1, 2, 7, 19, 8, True, 80), (2, 1, 16, 16, 8, True, 81),
                                              (1, 2, 23, 9, 16, False, 82), (1, 1, 1, 30, 8, True, 83)]:
        q, do = _rand((B, H, Nq, D), seed), _rand((B, H, Nq, D), seed + 3)
        k, v = _rand((B, H, Nk, D), seed + 1), _rand((B, H, Nk, D), seed + 2)
        scale = 0.3
        o, lse = fwd(q, k, v, causal, scale)
        tq, tk, tv = (torch.from_numpy(x).requires_grad_() for x in (q, k, v))
        mask = causal_lower_right(Nq, Nk) if causal else None
        ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask, scale=scale)
        np.testing.assert_allclose(o, ref.detach().numpy(), atol=tol)
        s = scale * (tq @ tk.transpose(-1, -2))
        if causal:
            s = s.masked_fill(~causal_lower_right(Nq, Nk)._materialize(), float("-inf"))
        np.testing.assert_allclose(lse, torch.logsumexp(s, dim=-1).detach().numpy(), atol=tol)
        ref.backward(torch.from_numpy(do))
        dq, dk, dv = bwd(q, k, v, do, causal, scale)
        for mine, theirs in ((dq, tq), (dk, tk), (dv, tv)):
            np.testing.assert_allclose(mine, theirs.grad.numpy(), atol=tol)


def pin_window_closed_forms(fwd, tol=1e-12):
    """Window 0 (causal) keeps only key i + N_k - N_q: O_i = v_that, lse_i = its score. A window
    covering every key is no window."""
    for (Nq, Nk) in [(13, 13), (5, 21)]:
        q, k, v = _rand((1, 2, Nq, 8), 90), _rand((1, 2, Nk, 8), 91), _rand((1, 2, Nk, 8), 92)
        off = Nk - Nq
        o, lse = fwd(q, k, v, True, 0.7, window=0)
        diag = np.arange(Nq) + off
        np.testing.assert_allclose(o, v[:, :, diag], atol=tol)
        np.testing.assert_allclose(lse, 0.7 * np.einsum("bhnd,bhnd->bhn", q, k[:, :, diag]), atol=tol)
        for causal in (False, True):
            o_w, lse_w = fwd(q, k, v, causal, 0.7, window=Nk + Nq)
            o_n, lse_n = fwd(q, k, v, causal, 0.7)
            np.testing.assert_allclose(o_w, o_n, atol=tol)
            np.testing.assert_allclose(lse_w, lse_n, atol=tol)


def pin_window_equals_key_slice(fwd, tol=1e-12):
    """Row i of windowed attention equals plain (unmasked) attention of q_i over the keys it keeps."""
    for (Nq, Nk, causal, w) in [(40, 40, True, 7), (11, 37, True, 15), (25, 25, False, 5)]:
        q, k, v = _rand((1, 1, Nq, 8), 100 + w), _rand((1, 1, Nk, 8), 101 + w), _rand((1, 1, Nk, 8), 102 + w)
        o, lse = fwd(q, k, v, causal, 0.5, window=w)
        for i in range(Nq):
            diag = i + Nk - Nq
            first = max(0, diag - w)
            last = min(Nk - 1, diag) if causal else Nk - 1
            ks, vs = k[:, :, first:last + 1], v[:, :, first:last + 1]
            o_i, lse_i = fwd(q[:, :, i:i + 1], ks, vs, False, 0.5)
            np.testing.assert_allclose(o[:, :, i:i + 1], o_i, atol=tol)
            np.testing.assert_allclose(lse[:, :, i:i + 1], lse_i, atol=tol)


def pin_brute_force_masks(fwd, bwd, brute, tol=1e-12):
    """The scalar-loop oracle with N_q != N_k and windows, forward and backward, on tiny heads."""
    for (Nq, Nk, causal, w, seed) in [(5, 9, True, 2, 110), (7, 7, True, 0, 111), (6, 4, False, 1, 112),
                                       (3, 11, True, -1, 113), (8, 8, False, 3, 114), (7, 3, True, -1, 115),
                                       (6, 4, True, 1, 116)]:
        q, do = _rand((1, 1, Nq, 4), seed), _rand((1, 1, Nq, 4), seed + 3)
        k, v = _rand((1, 1, Nk, 4), seed + 1), _rand((1, 1, Nk, 4), seed + 2)
        o, lse = fwd(q, k, v, causal, 0.6, window=w)
        o_b, lse_b = brute.forward(q[0, 0].tolist(), k[0, 0].tolist(), v[0, 0].tolist(), causal, 0.6, window=w)
        np.testing.assert_allclose(o[0, 0], np.array(o_b), atol=tol)
        np.testing.assert_allclose(lse[0, 0], np.array(lse_b), atol=tol)
        g = bwd(q, k, v, do, causal, 0.6, window=w)
        g_b = brute.backward(q[0, 0].tolist(), k[0, 0].tolist(), v[0, 0].tolist(), do[0, 0].tolist(), causal, 0.6,
                             window=w)
        for a, b in zip(g, g_b):
            np.testing.assert_allclose(a[0, 0], np.array(b), atol=tol)


def pin_finite_differences_masks(fwd, bwd, tol=1e-7):
    """Central differences of sum(dO * O) with N_q != N_k and a window match the backward."""
    q, do = _rand((1, 1, 4, 3), 120), _rand((1, 1, 4, 3), 123)
    k, v = _rand((1, 1, 7, 3), 121), _rand((1, 1, 7, 3), 122)
    causal, w, scale = True, 2, 0.8
    dq, dk, dv = bwd(q, k, v, do, causal, scale, window=w)
    eps = 1e-6
    for x, g in ((q, dq), (k, dk), (v, dv)):
        for idx in np.ndindex(x.shape):
            x0 = x[idx]
            x[idx] = x0 + eps
            lp = float((do * fwd(q, k, v, causal, scale, window=w)[0]).sum())
            x[idx] = x0 - eps
            lm = float((do * fwd(q, k, v, causal, scale, window=w)[0]).sum())
            x[idx] = x0
            assert abs((lp - lm) / (2 * eps) - g[idx]) <= tol, (idx, (lp - lm) / (2 * eps), g[idx])


FORWARD_PINS = [pin_zero_query, pin_constant_scores, pin_ones_value, pin_permutation, pin_key_shift,
                pin_scale_fold, pin_torch_forward]


def pin_empty_rows(fwd, bwd, tol=1e-11):
    """Causal with N_k < N_q: rows i < N_q - N_k keep no key -> O = 0, lse = -inf, zero dQ; the
    other rows are top-left causal attention of q[N_q - N_k:] (torch sdpa is_causal, a library
    routine). No keys at all: every row is empty."""
    import torch

    B, H, Nq, Nk, D = 1, 2, 9, 4, 8
    q, do = _rand((B, H, Nq, D), 130), _rand((B, H, Nq, D), 133)
    k, v = _rand((B, H, Nk, D), 131), _rand((B, H, Nk, D), 132)
    e = Nq - Nk
    o, lse = fwd(q, k, v, True, 0.45)
    assert np.all(o[:, :, :e] == 0.0) and np.all(lse[:, :, :e] == -np.inf)
    tq, tk, tv = (torch.from_numpy(x).requires_grad_() for x in (q[:, :, e:].copy(), k, v))
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=True, scale=0.45)
    np.testing.assert_allclose(o[:, :, e:], ref.detach().numpy(), atol=tol)
    s = 0.45 * (tq @ tk.transpose(-1, -2))
    s = s.masked_fill(torch.ones(Nk, Nk, dtype=torch.bool).triu(1), float("-inf"))
    np.testing.assert_allclose(lse[:, :, e:], torch.logsumexp(s, dim=-1).detach().numpy(), atol=tol)
    ref.backward(torch.from_numpy(do[:, :, e:].copy()))
    dq, dk, dv = bwd(q, k, v, do, True, 0.45)
    assert np.all(dq[:, :, :e] == 0.0)
    np.testing.assert_allclose(dq[:, :, e:], tq.grad.numpy(), atol=tol)
    np.testing.assert_allclose(dk, tk.grad.numpy(), atol=tol)
    np.testing.assert_allclose(dv, tv.grad.numpy(), atol=tol)
    # no keys at all
    o0, lse0 = fwd(q, k[:, :, :0], v[:, :, :0], False, 0.45)
    assert np.all(o0 == 0.0) and np.all(lse0 == -np.inf)


VARLEN_LENGTHS = [(5, 5), (0, 3), (7, 12), (4, 0), (1, 9), (6, 6), (9, 4)]


def pin_varlen_padded(fwd_varlen, bwd_varlen, tol=1e-11):
    """Packed sequences against torch sdpa + autograd on the zero-padded batch with a boolean mask
    built from each sequence's lengths (bottom-right causal, left window), grouped K/V heads."""
    import torch

    H, Hkv, D, scale = 4, 2, 8, 0.35
    nq = [a for a, _ in VARLEN_LENGTHS]
    nk = [b for _, b in VARLEN_LENGTHS]
    B, Lq, Lk = len(nq), max(nq), max(nk)
    cu_q, cu_k = np.concatenate([[0], np.cumsum(nq)]), np.concatenate([[0], np.cumsum(nk)])
    for causal, w, seed in [(False, -1, 140), (True, -1, 141), (True, 3, 142), (False, 2, 143)]:
        q, do = _rand((cu_q[-1], H, D), seed), _rand((cu_q[-1], H, D), seed + 3)
        k, v = _rand((cu_k[-1], Hkv, D), seed + 1), _rand((cu_k[-1], Hkv, D), seed + 2)
        o, lse = fwd_varlen(q, k, v, cu_q, cu_k, causal, scale, window=w)
        dq, dk, dv = bwd_varlen(q, k, v, do, cu_q, cu_k, causal, scale, window=w)
        # padded batch: [B, H, L, D], mask[b, i, j] True where query i of sequence b keeps key j
        pad = lambda x, cu, n, L, h: np.stack([np.pad(x[cu[b]:cu[b + 1]], ((0, L - n[b]), (0, 0), (0, 0)))
                                               for b in range(B)]).transpose(0, 2, 1, 3)
        qp, dop = pad(q, cu_q, nq, Lq, H), pad(do, cu_q, nq, Lq, H)
        kp, vp = pad(k, cu_k, nk, Lk, Hkv), pad(v, cu_k, nk, Lk, Hkv)
        i = np.arange(Lq)[:, None]
        j = np.arange(Lk)[None, :]
        mask = np.zeros((B, 1, Lq, Lk), dtype=bool)
        for b in range(B):
            keep = (i < nq[b]) & (j < nk[b])
            if causal:
                keep &= j <= i + nk[b] - nq[b]
            if w >= 0:
                keep &= j >= i + nk[b] - nq[b] - w
            mask[b, 0] = keep
        live = mask.any(axis=3)  # [B, 1, Lq]: rows that keep a key
        safe = mask.copy()
        safe[..., 0] |= ~live  # a dummy key for empty rows (their dO is zeroed below)
        tq, tk, tv = (torch.from_numpy(x).requires_grad_() for x in (qp, kp, vp))
        ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=torch.from_numpy(safe),
                                                               scale=scale, enable_gqa=True)
        g = H // Hkv
        s = scale * (tq @ tk.repeat_interleave(g, dim=1).transpose(-1, -2))
        lse_ref = torch.logsumexp(s.masked_fill(~torch.from_numpy(mask), float("-inf")), dim=-1)
        ref.backward(torch.from_numpy(dop * live[..., None]))
        for b in range(B):
            rows = slice(cu_q[b], cu_q[b + 1])
            lv = live[b, 0, :nq[b]]
            o_b = o[rows].transpose(1, 0, 2)       # [H, n, D]
            lse_b = lse[:, rows]
            np.testing.assert_allclose(o_b[:, lv], ref.detach().numpy()[b][:, :nq[b]][:, lv], atol=tol)
            np.testing.assert_allclose(lse_b[:, lv], lse_ref.detach().numpy()[b][:, :nq[b]][:, lv], atol=tol)
            assert np.all(o_b[:, ~lv] == 0.0) and np.all(lse_b[:, ~lv] == -np.inf)
            dq_b = dq[rows].transpose(1, 0, 2)
            np.testing.assert_allclose(dq_b[:, lv], tq.grad.numpy()[b][:, :nq[b]][:, lv], atol=tol)
            assert np.all(dq_b[:, ~lv] == 0.0)
            keys = slice(cu_k[b], cu_k[b + 1])
            np.testing.assert_allclose(dk[keys].transpose(1, 0, 2), tk.grad.numpy()[b][:, :nk[b]], atol=tol)
            np.testing.assert_allclose(dv[keys].transpose(1, 0, 2), tv.grad.numpy()[b][:, :nk[b]], atol=tol)


def _band(Nq, Nk, causal, w):
    i = np.arange(Nq)[:, None]
    j = np.arange(Nk)[None, :]
    keep = np.ones((Nq, Nk), dtype=bool)
    if causal:
        keep &= j <= i + Nk - Nq
    if w >= 0:
        keep &= j >= i + Nk - Nq - w
    return keep


def pin_block_mask_all_true(fwd, bwd, tol=1e-12):
    """A block mask that keeps every block is no mask."""
    q, do = _rand((1, 2, 37, 8), 150), _rand((1, 2, 37, 8), 153)
    k, v = _rand((1, 2, 45, 8), 151), _rand((1, 2, 45, 8), 152)
    for causal, block in ((False, 4), (True, 16), (True, 128)):
        m = np.ones((1, 2, -(-37 // block), -(-45 // block)), dtype=bool)
        o, lse = fwd(q, k, v, causal, 0.4, block_mask=m, block=block)
        o0, lse0 = fwd(q, k, v, causal, 0.4)
        np.testing.assert_allclose(o, o0, atol=tol)
        np.testing.assert_allclose(lse, lse0, atol=tol)
        for a, b in zip(bwd(q, k, v, do, causal, 0.4, block_mask=m, block=block), bwd(q, k, v, do, causal, 0.4)):
            np.testing.assert_allclose(a, b, atol=tol)


def pin_block_mask_torch(fwd, bwd, tol=1e-11):
    """torch CPU float64 sdpa + autograd with the boolean element mask kron(block_mask, ones) & band."""
    import torch

    for (B, H, Hkv, Nq, Nk, causal, w, block, seed) in [(1, 2, 2, 23, 30, False, -1, 4, 160),
                                                         (2, 4, 2, 19, 19, True, -1, 3, 161),
                                                         (1, 2, 1, 17, 29, True, 6, 5, 162)]:
        q, do = _rand((B, H, Nq, D := 8), seed), _rand((B, H, Nq, D), seed + 3)
        k, v = _rand((B, Hkv, Nk, D), seed + 1), _rand((B, Hkv, Nk, D), seed + 2)
        nqb, nkb = -(-Nq // block), -(-Nk // block)
        m = np.random.default_rng(seed + 4).random((B, H, nqb, nkb)) < 0.55
        o, lse = fwd(q, k, v, causal, 0.3, window=w, block_mask=m, block=block)
        dq, dk, dv = bwd(q, k, v, do, causal, 0.3, window=w, block_mask=m, block=block)
        elem = np.stack([np.stack([np.kron(m[b, h], np.ones((block, block), dtype=bool))[:Nq, :Nk]
                                   for h in range(H)]) for b in range(B)]) & _band(Nq, Nk, causal, w)
        live = elem.any(axis=3)
        safe = elem.copy()
        safe[..., 0] |= ~live  # a dummy key for empty rows, whose dO is zeroed
        tq, tk, tv = (torch.from_numpy(x).requires_grad_() for x in (q, k, v))
        ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=torch.from_numpy(safe),
                                                               scale=0.3, enable_gqa=True)
        s = 0.3 * (tq @ tk.repeat_interleave(H // Hkv, dim=1).transpose(-1, -2))
        lse_ref = torch.logsumexp(s.masked_fill(~torch.from_numpy(elem), float("-inf")), dim=-1)
        ref.backward(torch.from_numpy(do * live[..., None]))
        np.testing.assert_allclose(o[live], ref.detach().numpy()[live], atol=tol)
        np.testing.assert_allclose(lse[live], lse_ref.detach().numpy()[live], atol=tol)
        assert np.all(o[~live] == 0.0) and np.all(lse[~live] == -np.inf)
        np.testing.assert_allclose(dq, tq.grad.numpy(), atol=tol)
        np.testing.assert_allclose(dk, tk.grad.numpy(), atol=tol)
        np.testing.assert_allclose(dv, tv.grad.numpy(), atol=tol)


def pin_block_mask_drops_keys(fwd, tol=1e-12):
    """Without causal or window, masking key blocks out of every query block equals deleting those keys."""
    q = _rand((1, 1, 21, 8), 170)
    k, v = _rand((1, 1, 40, 8), 171), _rand((1, 1, 40, 8), 172)
    block = 8
    keep_blocks = np.array([True, False, True, True, False])
    m = np.broadcast_to(keep_blocks, (1, 1, 3, 5))
    o, lse = fwd(q, k, v, False, 0.6, block_mask=m, block=block)
    kept = np.repeat(keep_blocks, block)[:40]
    o2, lse2 = fwd(q, k[:, :, kept], v[:, :, kept], False, 0.6)
    np.testing.assert_allclose(o, o2, atol=tol)
    np.testing.assert_allclose(lse, lse2, atol=tol)


def pin_block_mask_brute(fwd, bwd, brute, tol=1e-12):
    """The scalar-loop oracle with a block mask, forward and backward."""
    for (Nq, Nk, causal, w, block, seed) in [(7, 9, False, -1, 2, 180), (8, 8, True, -1, 3, 181),
                                             (6, 10, True, 2, 2, 182)]:
        q, do = _rand((1, 1, Nq, 4), seed), _rand((1, 1, Nq, 4), seed + 3)
        k, v = _rand((1, 1, Nk, 4), seed + 1), _rand((1, 1, Nk, 4), seed + 2)
        m = np.random.default_rng(seed + 4).random((1, 1, -(-Nq // block), -(-Nk // block))) < 0.6
        o, lse = fwd(q, k, v, causal, 0.6, window=w, block_mask=m, block=block)
        ml = m[0, 0].tolist()
        o_b, lse_b = brute.forward(q[0, 0].tolist(), k[0, 0].tolist(), v[0, 0].tolist(), causal, 0.6, window=w,
                                   block_mask=ml, block=block)
        np.testing.assert_allclose(o[0, 0], np.array(o_b), atol=tol)
        np.testing.assert_allclose(lse[0, 0], np.array(lse_b), atol=tol)
        g = bwd(q, k, v, do, causal, 0.6, window=w, block_mask=m, block=block)
        g_b = brute.backward(q[0, 0].tolist(), k[0, 0].tolist(), v[0, 0].tolist(), do[0, 0].tolist(), causal, 0.6,
                             window=w, block_mask=ml, block=block)
        for a, b in zip(g, g_b):
            np.testing.assert_allclose(a[0, 0], np.array(b), atol=tol)


def pin_dq_rows_brute(dq_rows, brute, tol=1e-12):
    """The row-sampled dQ against pure-Python loops on N <= 16 (causal, window, N_q != N_k)."""
    for (nq, nk, causal, window, seed) in [(9, 9, False, -1, 80), (12, 7, True, -1, 81), (6, 14, True, 3, 82),
                                           (16, 16, True, 0, 83)]:
        q, do = (_rand((1, 1, nq, 5), seed + i) for i in range(2))
        k, v = (_rand((1, 1, nk, 5), seed + 2 + i) for i in range(2))
        rows = np.array(sorted({0, nq // 2, nq - 1}))
        got = dq_rows(q, k, v, do, causal, 0.8, rows, window=window)
        bdq, _, _ = brute.backward(q[0, 0].tolist(), k[0, 0].tolist(), v[0, 0].tolist(), do[0, 0].tolist(), causal,
                                   0.8, window=window)
        np.testing.assert_allclose(got[0, 0], np.array(bdq)[rows], atol=tol)


def pin_dq_rows_torch(dq_rows, tol=1e-11):
    """The row-sampled dQ against torch CPU float64 autograd of the plain formula (GQA, bottom-right causal)."""
    import torch

    B, H, Hkv, nq, nk, D = 2, 4, 2, 20, 33, 8
    q, do = (_rand((B, H, nq, D), 90 + i) for i in range(2))
    k, v = (_rand((B, Hkv, nk, D), 92 + i) for i in range(2))
    rows = np.array([0, 3, 11, 19])
    got = dq_rows(q, k, v, do, True, 0.45, rows)
    tq = torch.from_numpy(q).requires_grad_(True)
    tk = torch.from_numpy(k).repeat_interleave(H // Hkv, dim=1)
    tv = torch.from_numpy(v).repeat_interleave(H // Hkv, dim=1)
    s = 0.45 * (tq @ tk.transpose(-1, -2))
    i = torch.arange(nq)[:, None]
    j = torch.arange(nk)[None, :]
    s = s.masked_fill(j > i + (nk - nq), float("-inf"))
    (torch.softmax(s, dim=-1) @ tv * torch.from_numpy(do)).sum().backward()
    np.testing.assert_allclose(got, tq.grad.numpy()[:, :, rows], atol=tol)


def pin_kv_rows_brute(kv_rows, brute, tol=1e-12):
    """The row-sampled dK / dV against pure-Python loops on N <= 16 (causal, window, N_q != N_k)."""
    for (nq, nk, causal, window, seed) in [(9, 9, False, -1, 84), (12, 7, True, -1, 85), (6, 14, True, 3, 86),
                                           (16, 16, True, 0, 87), (7, 12, False, 2, 88)]:
        q, do = (_rand((1, 1, nq, 5), seed + i) for i in range(2))
        k, v = (_rand((1, 1, nk, 5), seed + 2 + i) for i in range(2))
        rows = np.array(sorted({0, 1, nk // 2, nk - 1}))
        gk, gv = kv_rows(q, k, v, do, causal, 0.8, rows, window=window)
        _, bdk, bdv = brute.backward(q[0, 0].tolist(), k[0, 0].tolist(), v[0, 0].tolist(), do[0, 0].tolist(),
                                     causal, 0.8, window=window)
        np.testing.assert_allclose(gk[0, 0], np.array(bdk)[rows], atol=tol)
        np.testing.assert_allclose(gv[0, 0], np.array(bdv)[rows], atol=tol)


def pin_kv_rows_torch(kv_rows, tol=1e-11):
    """The row-sampled dK / dV against torch CPU float64 autograd of the plain formula (GQA, bottom-right
    causal): a shared K/V head's gradients are the sums over its group."""
    import torch

    B, H, Hkv, nq, nk, D = 2, 4, 2, 20, 33, 8
    q, do = (_rand((B, H, nq, D), 94 + i) for i in range(2))
    k, v = (_rand((B, Hkv, nk, D), 96 + i) for i in range(2))
    rows = np.array([0, 5, 13, 14, 32])
    gk, gv = kv_rows(q, k, v, do, True, 0.45, rows)
    tk = torch.from_numpy(k).requires_grad_(True)
    tv = torch.from_numpy(v).requires_grad_(True)
    s = 0.45 * (torch.from_numpy(q) @ tk.repeat_interleave(H // Hkv, dim=1).transpose(-1, -2))
    i = torch.arange(nq)[:, None]
    j = torch.arange(nk)[None, :]
    s = s.masked_fill(j > i + (nk - nq), float("-inf"))
    (torch.softmax(s, dim=-1) @ tv.repeat_interleave(H // Hkv, dim=1) * torch.from_numpy(do)).sum().backward()
    np.testing.assert_allclose(gk, tk.grad.numpy()[:, :, rows], atol=tol)
    np.testing.assert_allclose(gv, tv.grad.numpy()[:, :, rows], atol=tol)
