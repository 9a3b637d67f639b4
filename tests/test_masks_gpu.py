"""GPU parity for query/key lengths that differ (bottom-right causal) and left sliding windows, through the C ABI.

Row i keeps keys j with i + (Nk - Nq) - window <= j <= i + (Nk - Nq) (lower bound only with a window, upper
bound only when causal). Compared element by element with the float64 oracle, whose masks are pinned to
torch's causal_lower_right bias, closed forms and per-row key slices.
"""
import math

import numpy as np
import pytest
import torch

from gpu_util import (REL_BF16, grad_err, TOL_BF16_GRAD, TOL_BF16_LSE, TOL_BF16_O, TOL_F32, max_abs, prepare, rel_fro,
                      sample_rows, to_f64)
from oracle import attention
from tiled_online_softmax_amd import fa, inputs

pytestmark = pytest.mark.gpu

VARIANTS = {"atomic": fa.FA_BWD_ATOMIC, "deterministic": fa.FA_BWD_DETERMINISTIC}
# (Nq, Nk, causal, window): lengths that differ, windows narrower and wider than a tile, both together
CASES = [(17, 80, True, None), (100, 333, True, None), (129, 64, False, None), (200, 200, True, 0),
         (300, 300, True, 31), (257, 257, True, 64), (130, 390, True, 100), (190, 190, False, 40),
         (64, 1000, True, 200), (1, 300, True, None), (1, 300, True, 5)]


def _win(w):
    return -1 if w is None else w


@pytest.mark.parametrize("Nq,Nk,causal,window", CASES)
@pytest.mark.parametrize("D", [64, 128])
def test_masks_fwd_bf16(Nq, Nk, causal, window, D):
    dev, ref = prepare("bf16", (2, 4, Nq, D), 4000 + Nq + Nk + D + _win(window), hkv=2, nk=Nk)
    scale = 1.0 / math.sqrt(D)
    o, lse = fa.fwd(dev["q"], dev["k"], dev["v"], causal=causal, scale=scale, window=window)
    o_ref, lse_ref = attention.forward(ref["q"], ref["k"], ref["v"], causal, scale, window=_win(window))
    eo, el = max_abs(to_f64(o), o_ref), max_abs(to_f64(lse), lse_ref)
    print(f"[masks fwd Nq{Nq} Nk{Nk} causal={causal} w={window} D{D}] O {eo:.3e} lse {el:.3e}", flush=True)
    assert eo <= TOL_BF16_O and el <= TOL_BF16_LSE


@pytest.mark.parametrize("Nq,Nk,causal,window", [(33, 97, True, None), (150, 150, True, 20), (90, 40, False, 7)])
def test_masks_fwd_f32(Nq, Nk, causal, window):
    dev, ref = prepare("f32", (1, 2, Nq, 64), 4100 + Nq, nk=Nk)
    o, lse = fa.fwd(dev["q"], dev["k"], dev["v"], causal=causal, scale=0.125, window=window)
    o_ref, lse_ref = attention.forward(ref["q"], ref["k"], ref["v"], causal, 0.125, window=_win(window))
    assert max_abs(to_f64(o), o_ref) <= TOL_F32 and max_abs(to_f64(lse), lse_ref) <= TOL_F32


def test_window_zero_keeps_the_diagonal_key():
    """With window 0 each row keeps only its diagonal key: O_i = v_(i+Nk-Nq) up to bf16 rounding of O."""
    dev, ref = prepare("bf16", (1, 2, 150, 128), 4200, nk=400)
    o, _ = fa.fwd(dev["q"], dev["k"], dev["v"], causal=True, window=0)
    diag = np.arange(150) + 250
    assert max_abs(to_f64(o), ref["v"][:, :, diag]) <= 2 ** -8 * np.abs(ref["v"]).max()


def test_full_window_equals_no_window():
    dev, _ = prepare("bf16", (1, 4, 300, 128), 4300, nk=700)
    o, lse = fa.fwd(dev["q"], dev["k"], dev["v"], causal=True)
    o_w, lse_w = fa.fwd(dev["q"], dev["k"], dev["v"], causal=True, window=10_000)
    torch.cuda.synchronize()
    assert max_abs(to_f64(o), to_f64(o_w)) <= 2e-2 and max_abs(to_f64(lse), to_f64(lse_w)) <= 1e-5


def _check_grads(g, g_ref, tag, group=1):
    errs = [grad_err(a, b) for a, b in zip(g, g_ref)]
    rels = [rel_fro(a, b) for a, b in zip(g, g_ref)]
    tols = [TOL_BF16_GRAD, TOL_BF16_GRAD * math.sqrt(group), TOL_BF16_GRAD * math.sqrt(group)]
    print(f"[{tag}] max(|d|-ulp) dQ={errs[0]:.3e} dK={errs[1]:.3e} dV={errs[2]:.3e} rel={max(rels):.3e}", flush=True)
    assert all(e <= t for e, t in zip(errs, tols)), (tag, errs, tols)
    if g[0].shape[2] >= 64:
        assert max(rels) <= 2e-2, (tag, rels)


@pytest.mark.parametrize("variant", sorted(VARIANTS))
@pytest.mark.parametrize("Nq,Nk,causal,window", CASES)
@pytest.mark.parametrize("D", [64, 128])
def test_masks_bwd(variant, Nq, Nk, causal, window, D):
    dev, ref = prepare("bf16", (1, 4, Nq, D), 4400 + Nq + Nk + D + _win(window), with_grad=True, hkv=2, nk=Nk)
    scale = 1.0 / math.sqrt(D)
    o, lse = fa.fwd(dev["q"], dev["k"], dev["v"], causal=causal, scale=scale, window=window)
    g = fa.bwd(dev["q"], dev["k"], dev["v"], o, dev["do"], lse, causal=causal, scale=scale,
               variant=VARIANTS[variant], window=window)
    torch.cuda.synchronize()
    g_ref = attention.backward(ref["q"], ref["k"], ref["v"], ref["do"], causal, scale, window=_win(window))
    _check_grads([to_f64(x) for x in g], g_ref, f"masks bwd {variant} Nq{Nq} Nk{Nk} c={causal} w={window} D{D}", 2)


def test_keys_no_query_keeps_get_zero_gradients():
    """Non-causal window 10 with Nq = 50, Nk = 400: keys below 340 - 10 are kept by no row."""
    dev, ref = prepare("bf16", (1, 2, 50, 64), 4500, with_grad=True, nk=400)
    o, lse = fa.fwd(dev["q"], dev["k"], dev["v"], causal=False, window=10)
    for variant in VARIANTS.values():
        dq, dk, dv = fa.bwd(dev["q"], dev["k"], dev["v"], o, dev["do"], lse, causal=False, variant=variant,
                            window=10)
        torch.cuda.synchronize()
        assert not dk[:, :, :340].any() and not dv[:, :, :340].any()
        g_ref = attention.backward(ref["q"], ref["k"], ref["v"], ref["do"], False, 0.125, window=10)
        _check_grads([to_f64(x) for x in (dq, dk, dv)], g_ref, "unkept keys")


@pytest.mark.parametrize("name", ["prefill_bf16", "swa_bf16"])
def test_workload_fwd_sampled_rows(name):
    """Full-size forward in the launch bench.py times; sampled rows of every head against the oracle."""
    w = inputs.WORKLOADS[name]
    dev, ref = prepare("bf16", w.shape, w.seed, nk=w.nk)
    o, lse = fa.fwd(dev["q"], dev["k"], dev["v"], causal=w.causal, window=w.window)
    torch.cuda.synchronize()
    rows = sample_rows(w.N)
    o_ref, lse_ref = attention.forward(ref["q"], ref["k"], ref["v"], w.causal, w.scale, rows=rows,
                                       window=_win(w.window))
    og, lg = to_f64(o)[:, :, rows], to_f64(lse)[:, :, rows]
    eo, el, rf = max_abs(og, o_ref), max_abs(lg, lse_ref), rel_fro(og, o_ref)
    print(f"[{name} fwd] O {eo:.3e} lse {el:.3e} rel {rf:.3e}", flush=True)
    assert eo <= TOL_BF16_O and el <= TOL_BF16_LSE and rf <= REL_BF16


@pytest.mark.parametrize("name", ["prefill_bf16", "swa_bf16"])
def test_workload_bwd_two_heads(name):
    """Full-size backward; every element of two heads against the oracle."""
    w = inputs.WORKLOADS[name]
    dev, ref = prepare("bf16", w.shape, w.seed, with_grad=True, nk=w.nk)
    o, lse = fa.fwd(dev["q"], dev["k"], dev["v"], causal=w.causal, window=w.window)
    g = fa.bwd(dev["q"], dev["k"], dev["v"], o, dev["do"], lse, causal=w.causal, variant=fa.FA_BWD_DETERMINISTIC,
               window=w.window)
    torch.cuda.synchronize()
    for b, h in ((0, 0), (w.B - 1, w.H - 1)):
        sl = (slice(b, b + 1), slice(h, h + 1))
        g_ref = attention.backward(ref["q"][sl], ref["k"][sl], ref["v"][sl], ref["do"][sl], w.causal, w.scale,
                                   window=_win(w.window))
        _check_grads([to_f64(x[sl]) for x in g], g_ref, f"{name} bwd b{b} h{h}")
