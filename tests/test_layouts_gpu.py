"""GPU parity: strided layouts, packed variable-length batches, and rows that keep no key.

Strided calls go through fa_fwd_strided / fa_bwd_strided (any batch, head and row strides, D
contiguous). They run the same kernels as the contiguous entry points with other addresses, so
besides the oracle comparison each case must equal the contiguous call bitwise (the atomics-free
backward; the atomic one only within tolerance, its float atomics add in any order). Packed
sequences (fa_fwd_varlen / fa_bwd_varlen) are compared with the oracle's per-sequence definition
and, bitwise, with one fa_fwd_general call per sequence.
"""
from __future__ import annotations

import math

import numpy as np
import pytest
import torch

from gpu_util import (DEV, TOL_BF16_GRAD, grad_err, TOL_BF16_LSE, TOL_BF16_O, TOL_F32, max_abs, prepare, rel_fro,
                      to_f64)
from oracle import attention
from tiled_online_softmax_amd import fa

pytestmark = pytest.mark.gpu

VARIANTS = {"atomic": fa.FA_BWD_ATOMIC, "deterministic": fa.FA_BWD_DETERMINISTIC}


def _bnhd(t: torch.Tensor) -> torch.Tensor:
    """The same values as the contiguous [B, H, N, D] tensor t, stored as [B, N, H, D] and viewed back."""
    return t.transpose(1, 2).contiguous().transpose(1, 2)


def _packed_qkv(q, k, v):
    """Views of one [B, N, 3, H, D] buffer holding q, k, v (the output layout of a fused QKV projection)."""
    B, H, N, D = q.shape
    buf = torch.empty((B, N, 3, H, D), dtype=q.dtype, device=q.device)
    for i, t in enumerate((q, k, v)):
        buf[:, :, i] = t.transpose(1, 2)
    return tuple(buf[:, :, i].transpose(1, 2) for i in range(3))


def _win(w):
    return -1 if w is None else w


def _same(a: torch.Tensor, b: torch.Tensor) -> bool:
    return torch.equal(a.contiguous().view(torch.int16 if a.dtype == torch.bfloat16 else a.dtype),
                       b.contiguous().view(torch.int16 if b.dtype == torch.bfloat16 else b.dtype))


# (dtype, B, H, Hkv, Nq, Nk, D, causal, window)
FWD_CASES = [("bf16", 2, 4, 4, 200, 200, 128, True, None), ("bf16", 2, 4, 2, 129, 300, 64, True, None),
             ("bf16", 1, 4, 1, 300, 300, 256, False, None), ("bf16", 2, 4, 2, 257, 257, 128, True, 40),
             ("f32", 1, 2, 2, 100, 170, 64, False, None), ("f32", 1, 2, 1, 150, 150, 128, True, 20)]


@pytest.mark.parametrize("case", FWD_CASES, ids=lambda c: "-".join(map(str, c)))
def test_strided_fwd_bnhd(case):
    dt, B, H, Hkv, Nq, Nk, D, causal, window = case
    dev, ref = prepare(dt, (B, H, Nq, D), 6000 + Nq + Nk + D, hkv=Hkv, nk=Nk)
    q, k, v = (_bnhd(dev[n]) for n in ("q", "k", "v"))
    assert not q.is_contiguous()
    out = _bnhd(torch.empty((B, H, Nq, D), dtype=torch.float32 if dt == "f32" else torch.bfloat16, device=DEV))
    o, lse = fa.fwd(q, k, v, causal=causal, window=window, out=out)
    o_c, lse_c = fa.fwd(dev["q"], dev["k"], dev["v"], causal=causal, window=window)
    torch.cuda.synchronize()
    assert _same(o, o_c) and _same(lse, lse_c), "strided forward differs from the contiguous one"
    o_ref, lse_ref = attention.forward(ref["q"], ref["k"], ref["v"], causal, 1 / math.sqrt(D), window=_win(window))
    eo, el = max_abs(to_f64(o), o_ref), max_abs(to_f64(lse), lse_ref)
    print(f"[strided fwd {case}] O {eo:.3e} lse {el:.3e}", flush=True)
    tol_o, tol_l = (TOL_F32, TOL_F32) if dt == "f32" else (TOL_BF16_O, TOL_BF16_LSE)
    assert eo <= tol_o and el <= tol_l


@pytest.mark.parametrize("D", [64, 128])
def test_strided_fwd_packed_qkv_and_mixed_row_strides(D):
    """Q, K, V as views of one fused-projection buffer (rows 3*H*D apart), and K from that buffer with
    V contiguous (K and V rows spaced differently, read through one tile loader)."""
    B, H, N = 2, 4, 333
    dev, ref = prepare("bf16", (B, H, N, D), 6100 + D)
    q, k, v = _packed_qkv(dev["q"], dev["k"], dev["v"])
    o_c, lse_c = fa.fwd(dev["q"], dev["k"], dev["v"], causal=True)
    o1, lse1 = fa.fwd(q, k, v, causal=True)
    o2, lse2 = fa.fwd(q, k, dev["v"], causal=True)
    o3, lse3 = fa.fwd(dev["q"], dev["k"], v, causal=True)
    torch.cuda.synchronize()
    for o, lse in ((o1, lse1), (o2, lse2), (o3, lse3)):
        assert _same(o, o_c) and _same(lse, lse_c)
    o_ref, lse_ref = attention.forward(ref["q"], ref["k"], ref["v"], True, 1 / math.sqrt(D))
    assert max_abs(to_f64(o1), o_ref) <= TOL_BF16_O and max_abs(to_f64(lse1), lse_ref) <= TOL_BF16_LSE


@pytest.mark.parametrize("variant", sorted(VARIANTS))
@pytest.mark.parametrize("case", [(2, 4, 4, 200, 200, 128, True, None), (1, 4, 2, 129, 300, 64, True, None),
                                  (2, 4, 2, 257, 257, 128, True, 40), (1, 4, 4, 190, 190, 64, False, None)],
                         ids=lambda c: "-".join(map(str, c)))
def test_strided_bwd(variant, case):
    B, H, Hkv, Nq, Nk, D, causal, window = case
    dev, ref = prepare("bf16", (B, H, Nq, D), 6200 + Nq + Nk + D, with_grad=True, hkv=Hkv, nk=Nk)
    o_c, lse_c = fa.fwd(dev["q"], dev["k"], dev["v"], causal=causal, window=window)
    g_c = fa.bwd(dev["q"], dev["k"], dev["v"], o_c, dev["do"], lse_c, causal=causal, window=window,
                 variant=VARIANTS[variant])
    q, k, v, o, do = (_bnhd(t) for t in (dev["q"], dev["k"], dev["v"], o_c, dev["do"]))
    grads = [_bnhd(torch.empty_like(t)) for t in (dev["q"], dev["k"], dev["v"])]
    g = fa.bwd(q, k, v, o, do, lse_c, causal=causal, window=window, variant=VARIANTS[variant], dq=grads[0],
               dk=grads[1], dv=grads[2])
    torch.cuda.synchronize()
    if variant == "deterministic":
        assert all(_same(a, b) for a, b in zip(g, g_c)), "strided backward differs from the contiguous one"
    g_ref = attention.backward(ref["q"], ref["k"], ref["v"], ref["do"], causal, 1 / math.sqrt(D),
                               window=_win(window))
    errs = [grad_err(to_f64(a), b) for a, b in zip(g, g_ref)]
    tol = [TOL_BF16_GRAD, TOL_BF16_GRAD * math.sqrt(H // Hkv), TOL_BF16_GRAD * math.sqrt(H // Hkv)]
    print(f"[strided bwd {variant} {case}] dQ {errs[0]:.3e} dK {errs[1]:.3e} dV {errs[2]:.3e}", flush=True)
    assert all(e <= t for e, t in zip(errs, tol))


# Sequence lengths (queries, keys) of a packed batch: empty sequences on either side, lengths
# below, at and across tile sizes, fewer keys than queries.
LENGTHS = [(70, 70), (0, 20), (129, 300), (5, 0), (1, 64), (256, 256), (200, 100), (33, 513)]


def _packed(lengths, H, Hkv, D, seed, with_grad=False):
    nq = np.array([a for a, _ in lengths])
    nk = np.array([b for _, b in lengths])
    cu_q = np.concatenate([[0], np.cumsum(nq)]).astype(np.int32)
    cu_k = np.concatenate([[0], np.cumsum(nk)]).astype(np.int32)
    dev, ref = prepare("bf16", (int(cu_q[-1]), H, D), seed, with_grad=with_grad, kv_shape=(int(cu_k[-1]), Hkv, D))
    return dev, ref, cu_q, cu_k, int(nq.max()), int(nk.max())


@pytest.mark.parametrize("causal,window", [(False, None), (True, None), (True, 50)])
@pytest.mark.parametrize("D", [64, 128])
def test_varlen_fwd(causal, window, D):
    H, Hkv = 4, 2
    dev, ref, cu_q, cu_k, mq, mk = _packed(LENGTHS, H, Hkv, D, 6300 + D)
    tq, tk = (torch.from_numpy(c).to(DEV) for c in (cu_q, cu_k))
    o, lse = fa.fwd_varlen(dev["q"], dev["k"], dev["v"], tq, tk, mq, mk, causal=causal, window=window)
    torch.cuda.synchronize()
    o_ref, lse_ref = attention.forward_varlen(ref["q"], ref["k"], ref["v"], cu_q, cu_k, causal, 1 / math.sqrt(D),
                                              window=_win(window))
    og, lg = to_f64(o), to_f64(lse)
    empty = lse_ref == -np.inf
    assert np.all(lg[empty] == -np.inf) and np.all(og.transpose(1, 0, 2)[empty] == 0.0)
    eo, el = max_abs(og, o_ref), max_abs(lg[~empty], lse_ref[~empty])
    print(f"[varlen fwd causal={causal} w={window} D{D}] O {eo:.3e} lse {el:.3e}", flush=True)
    assert eo <= TOL_BF16_O and el <= TOL_BF16_LSE
    # bitwise: one fa_fwd_general call per sequence
    for b in range(len(LENGTHS)):
        qs, ks = slice(cu_q[b], cu_q[b + 1]), slice(cu_k[b], cu_k[b + 1])
        if cu_q[b + 1] == cu_q[b] or cu_k[b + 1] == cu_k[b]:
            continue
        per = lambda t, s: t[s].transpose(0, 1).unsqueeze(0).contiguous()
        o_b, lse_b = fa.fwd(per(dev["q"], qs), per(dev["k"], ks), per(dev["v"], ks), causal=causal, window=window)
        torch.cuda.synchronize()
        assert _same(o[qs], o_b[0].transpose(0, 1)) and _same(lse[:, qs], lse_b[0]), b


@pytest.mark.parametrize("variant", sorted(VARIANTS))
@pytest.mark.parametrize("causal,window", [(False, None), (True, None), (True, 50)])
def test_varlen_bwd(variant, causal, window):
    H, Hkv, D = 4, 2, 128
    dev, ref, cu_q, cu_k, mq, mk = _packed(LENGTHS, H, Hkv, D, 6400 + int(causal), with_grad=True)
    tq, tk = (torch.from_numpy(c).to(DEV) for c in (cu_q, cu_k))
    o, lse = fa.fwd_varlen(dev["q"], dev["k"], dev["v"], tq, tk, mq, mk, causal=causal, window=window)
    g = fa.bwd_varlen(dev["q"], dev["k"], dev["v"], o, dev["do"], lse, tq, tk, mq, mk, causal=causal,
                      window=window, variant=VARIANTS[variant])
    torch.cuda.synchronize()
    g_ref = attention.backward_varlen(ref["q"], ref["k"], ref["v"], ref["do"], cu_q, cu_k, causal,
                                      1 / math.sqrt(D), window=_win(window))
    errs = [grad_err(to_f64(a), b) for a, b in zip(g, g_ref)]
    rels = [rel_fro(to_f64(a), b) for a, b in zip(g, g_ref)]
    print(f"[varlen bwd {variant} causal={causal} w={window}] dQ {errs[0]:.3e} dK {errs[1]:.3e} "
          f"dV {errs[2]:.3e} rel {max(rels):.3e}", flush=True)
    g2 = TOL_BF16_GRAD * math.sqrt(H // Hkv)
    assert errs[0] <= TOL_BF16_GRAD and errs[1] <= g2 and errs[2] <= g2 and max(rels) <= 2e-2
    if variant == "deterministic":
        g_again = fa.bwd_varlen(dev["q"], dev["k"], dev["v"], o, dev["do"], lse, tq, tk, mq, mk, causal=causal,
                                window=window, variant=VARIANTS[variant])
        torch.cuda.synchronize()
        assert all(_same(a, b) for a, b in zip(g, g_again))


@pytest.mark.parametrize("D", [64, 128])
def test_rows_without_keys(D):
    """Causal with Nk < Nq: rows i < Nq - Nk keep no key -> O = 0, lse = -inf, dQ = 0; the rest match the oracle."""
    B, H, Nq, Nk = 1, 4, 300, 130
    dev, ref = prepare("bf16", (B, H, Nq, D), 6500 + D, with_grad=True, hkv=2, nk=Nk)
    o, lse = fa.fwd(dev["q"], dev["k"], dev["v"], causal=True)
    torch.cuda.synchronize()
    e = Nq - Nk
    og, lg = to_f64(o), to_f64(lse)
    assert np.all(og[:, :, :e] == 0.0) and np.all(lg[:, :, :e] == -np.inf)
    o_ref, lse_ref = attention.forward(ref["q"], ref["k"], ref["v"], True, 1 / math.sqrt(D))
    assert max_abs(og, o_ref) <= TOL_BF16_O and max_abs(lg[:, :, e:], lse_ref[:, :, e:]) <= TOL_BF16_LSE
    g_ref = attention.backward(ref["q"], ref["k"], ref["v"], ref["do"], True, 1 / math.sqrt(D))
    for variant in VARIANTS.values():
        g = fa.bwd(dev["q"], dev["k"], dev["v"], o, dev["do"], lse, causal=True, variant=variant)
        torch.cuda.synchronize()
        assert not g[0][:, :, :e].any()
        errs = [grad_err(to_f64(a), b) for a, b in zip(g, g_ref)]
        assert errs[0] <= TOL_BF16_GRAD and max(errs[1:]) <= TOL_BF16_GRAD * math.sqrt(2), errs
    # the f32 forward and a query tile whose rows all keep no key
    dev32, ref32 = prepare("f32", (1, 2, 200, 64), 6510, nk=40)
    o32, lse32 = fa.fwd(dev32["q"], dev32["k"], dev32["v"], causal=True)
    torch.cuda.synchronize()
    o_ref, lse_ref = attention.forward(ref32["q"], ref32["k"], ref32["v"], True, 0.125)
    assert np.all(to_f64(lse32)[:, :, :160] == -np.inf) and max_abs(to_f64(o32), o_ref) <= TOL_F32


def test_workload_varlen_bf16():
    """The packed 16-sequence workload at full size, as the bench launches it: forward rows of five sequences
    (the four shortest in full, sampled rows of the longest) and the backward of the shortest three."""
    from tiled_online_softmax_amd import inputs
    from gpu_util import sample_rows
    w = inputs.WORKLOADS["varlen_bf16"]
    dev, ref = prepare("bf16", w.shape, w.seed, with_grad=True, kv_shape=w.kv_shape)
    cu = w.cu_seqlens()
    tcu = torch.from_numpy(cu).to(DEV)
    mx = max(w.lengths)
    o, lse = fa.fwd_varlen(dev["q"], dev["k"], dev["v"], tcu, tcu, mx, mx, causal=True)
    g = fa.bwd_varlen(dev["q"], dev["k"], dev["v"], o, dev["do"], lse, tcu, tcu, mx, mx, causal=True,
                      variant=fa.FA_BWD_DETERMINISTIC)
    torch.cuda.synchronize()
    og, lg = to_f64(o), to_f64(lse)
    for b in (0, 12, 13, 14, 15):
        s = slice(cu[b], cu[b + 1])
        n = cu[b + 1] - cu[b]
        rows = sample_rows(n) if n > 1024 else np.arange(n)
        t = lambda x: x[s].transpose(1, 0, 2)[None]
        o_ref, lse_ref = attention.forward(t(ref["q"]), t(ref["k"]), t(ref["v"]), True, w.scale, rows=rows)
        eo = max_abs(og[s][rows].transpose(1, 0, 2)[None], o_ref)
        el = max_abs(lg[:, s][:, rows][None], lse_ref)
        print(f"[varlen workload seq {b} n={n}] O {eo:.3e} lse {el:.3e}", flush=True)
        assert eo <= TOL_BF16_O and el <= TOL_BF16_LSE
    for b in (13, 14, 15):
        s = slice(cu[b], cu[b + 1])
        t = lambda x: x[s].transpose(1, 0, 2)[None]
        g_ref = attention.backward(t(ref["q"]), t(ref["k"]), t(ref["v"]), t(ref["do"]), True, w.scale)
        for a, r in zip(g, g_ref):
            assert grad_err(to_f64(a)[s].transpose(1, 0, 2)[None], r) <= TOL_BF16_GRAD
