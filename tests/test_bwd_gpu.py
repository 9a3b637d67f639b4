"""GPU parity of the backward kernels (bf16) against the float64 oracle, through the C ABI.

The GPU backward consumes the GPU forward's bf16 O and float32 lse; the
oracle returns the exact gradient at the same bf16 inputs (its own float64
forward), so forward rounding enters only through D_i = rowsum(dO * O).
"""
import math

import numpy as np
import pytest
import torch

from gpu_util import TOL_BF16_GRAD, grad_err, max_abs, prepare, rel_fro, to_f64
from gpu_util import sample_rows
from oracle import attention
from tiled_online_softmax_amd import fa, inputs

pytestmark = pytest.mark.gpu

VARIANTS = {"atomic": fa.FA_BWD_ATOMIC, "deterministic": fa.FA_BWD_DETERMINISTIC}


def _grads(dev, causal, scale, variant):
    o, lse = fa.fwd(dev["q"], dev["k"], dev["v"], causal=causal, scale=scale)
    g = fa.bwd(dev["q"], dev["k"], dev["v"], o, dev["do"], lse, causal=causal, scale=scale, variant=variant)
    torch.cuda.synchronize()
    return [to_f64(x) for x in g]


def _check(g, g_ref, tag, tol=TOL_BF16_GRAD):
    errs = [grad_err(a, b) for a, b in zip(g, g_ref)]
    rels = [rel_fro(a, b) for a, b in zip(g, g_ref)]
    print(f"[{tag}] max(|d|-ulp) dQ={errs[0]:.3e} dK={errs[1]:.3e} dV={errs[2]:.3e} rel={max(rels):.3e}", flush=True)
    assert max(errs) <= tol, (tag, errs)
    # The relative diagnostic guards against near-zero outputs passing the absolute bound on
    # large problems; on a handful of rows (N < 64) dQ and dK are themselves near zero
    # (cancellation in dS), so a relative measure there is meaningless.
    if g[0].shape[2] >= 64:
        assert max(rels) <= 2e-2, (tag, rels)


@pytest.mark.parametrize("variant", sorted(VARIANTS))
def test_bwd_causal_workload_full(variant):
    """B=2 H=16 N=4096 D=64 bf16 causal, every element of dQ, dK, dV."""
    w = inputs.WORKLOADS["bwd_causal_bf16"]
    dev, ref = prepare("bf16", w.shape, w.seed, with_grad=True)
    g = _grads(dev, w.causal, w.scale, VARIANTS[variant])
    g_ref = attention.backward(ref["q"], ref["k"], ref["v"], ref["do"], w.causal, w.scale)
    _check(g, g_ref, f"{w.name} {variant}")


@pytest.mark.parametrize("variant", sorted(VARIANTS))
@pytest.mark.parametrize("D", [64, 128, 256])
@pytest.mark.parametrize("causal", [False, True])
def test_bwd_small_shapes(variant, D, causal):
    for i, N in enumerate([1, 2, 17, 28, 29, 30, 31, 63, 65, 129, 300]):
        dev, ref = prepare("bf16", (1, 2, N, D), 2000 + 31 * i + D, with_grad=True)
        scale = 1.0 / math.sqrt(D)
        g = _grads(dev, causal, scale, VARIANTS[variant])
        g_ref = attention.backward(ref["q"], ref["k"], ref["v"], ref["do"], causal, scale)
        _check(g, g_ref, f"{variant} D{D} N{N} causal={causal}")


@pytest.mark.parametrize("variant", sorted(VARIANTS))
def test_bwd_multi_batch_head(variant):
    dev, ref = prepare("bf16", (2, 3, 333, 128), 88, with_grad=True)
    scale = 1.0 / math.sqrt(128)
    g = _grads(dev, True, scale, VARIANTS[variant])
    g_ref = attention.backward(ref["q"], ref["k"], ref["v"], ref["do"], True, scale)
    _check(g, g_ref, f"{variant} B2 H3 N333")


def test_bwd_identities_on_gpu():
    """sum_j dK_j = 0 and sum_j dV_j = sum_i dO_i hold for the exact gradient; the GPU must follow."""
    dev, ref = prepare("bf16", (1, 4, 1000, 64), 99, with_grad=True)
    for variant in VARIANTS.values():
        dq, dk, dv = _grads(dev, True, 0.125, variant)
        assert np.abs(dk.sum(axis=2)).max() <= 0.1
        assert max_abs(dv.sum(axis=2), ref["do"].sum(axis=2)) <= 0.1


def test_deterministic_variant_is_bitwise_stable():
    dev, _ = prepare("bf16", (1, 4, 777, 64), 5, with_grad=True)
    o, lse = fa.fwd(dev["q"], dev["k"], dev["v"], causal=True)
    ref = fa.bwd(dev["q"], dev["k"], dev["v"], o, dev["do"], lse, causal=True, variant=fa.FA_BWD_DETERMINISTIC)
    for _ in range(5):
        g = fa.bwd(dev["q"], dev["k"], dev["v"], o, dev["do"], lse, causal=True, variant=fa.FA_BWD_DETERMINISTIC)
        for a, b in zip(g, ref):
            assert torch.equal(a, b)


@pytest.mark.parametrize("D", [128, 256])
def test_variants_agree(D):
    dev, _ = prepare("bf16", (1, 2, 900, D), 6, with_grad=True)
    ga = _grads(dev, True, 0.1, fa.FA_BWD_ATOMIC)
    gd = _grads(dev, True, 0.1, fa.FA_BWD_DETERMINISTIC)
    # The variants use different key-pass tilings and query-tile orders, so dK and dV differ only by
    # the fp32 summation order: at most one bf16 step of the larger value, up to cancellation near zero.
    for a, b in ((ga[1], gd[1]), (ga[2], gd[2])):
        a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
        bound = 2.0 ** -7 * np.maximum(np.abs(a), np.abs(b)) + 1e-4 * np.abs(a).max()
        assert np.all(np.abs(a - b) <= bound)
    assert max_abs(ga[0], gd[0]) <= 1e-2


def test_dkdv_only_matches_full_backward():
    """fa_bwd_dkdv returns bitwise the dK, dV of fa_bwd."""
    dev, _ = prepare("bf16", (2, 3, 700, 128), 21, with_grad=True)
    for causal in (False, True):
        o, lse = fa.fwd(dev["q"], dev["k"], dev["v"], causal=causal)
        _, dk, dv = fa.bwd(dev["q"], dev["k"], dev["v"], o, dev["do"], lse, causal=causal,
                           variant=fa.FA_BWD_DETERMINISTIC)
        dk2, dv2 = fa.bwd_dkdv(dev["q"], dev["k"], dev["v"], o, dev["do"], lse, causal=causal)
        torch.cuda.synchronize()
        assert torch.equal(dk, dk2) and torch.equal(dv, dv2)


_D256_REF = {}


@pytest.mark.parametrize("variant", sorted(VARIANTS))
def test_bwd_d256_causal_workload(variant):
    """B=1 H=8 N=8192 D=256 bf16 x0.5 causal (the large-head-dim workload's shape and values, causal): dQ on
    sampled rows of every head, and every element of dQ, dK and dV of two heads."""
    w = inputs.WORKLOADS["bwd_d256_bf16"]
    dev, ref = prepare("bf16", w.shape, w.seed, w.multiplier, with_grad=True)
    o, lse = fa.fwd(dev["q"], dev["k"], dev["v"], causal=w.causal, scale=w.scale)
    dq, dk, dv = fa.bwd(dev["q"], dev["k"], dev["v"], o, dev["do"], lse, causal=w.causal, scale=w.scale,
                        variant=VARIANTS[variant])
    torch.cuda.synchronize()
    rows = sample_rows(w.N)
    if "dq_rows" not in _D256_REF:
        _D256_REF["dq_rows"] = attention.backward_dq_rows(ref["q"], ref["k"], ref["v"], ref["do"], w.causal, w.scale,
                                                          rows)
    e = grad_err(to_f64(dq)[:, :, rows], _D256_REF["dq_rows"])
    print(f"[{w.name} {variant}] dQ on {len(rows)} rows of every head: {e:.3e}", flush=True)
    assert e <= TOL_BF16_GRAD
    for h in (0, 5):
        sl = (slice(0, 1), slice(h, h + 1))
        if h not in _D256_REF:
            _D256_REF[h] = attention.backward(ref["q"][sl], ref["k"][sl], ref["v"][sl], ref["do"][sl], w.causal,
                                              w.scale)
        _check([to_f64(x)[sl] for x in (dq, dk, dv)], _D256_REF[h], f"{w.name} {variant} head {h}")
