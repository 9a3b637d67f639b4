"""GPU parity of grouped-query attention (K/V heads shared by groups of query heads) through the C ABI.

Query head h uses K/V head h // (H / Hkv); the backward sums a shared K/V
head's dK and dV over its group. Compared against the float64 oracle, whose
grouped-query form is pinned to torch's scaled_dot_product_attention with
enable_gqa on the CPU.
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
GROUPS = [(4, 1), (4, 2), (6, 3), (8, 2)]  # (query heads, K/V heads)


@pytest.mark.parametrize("H,Hkv", GROUPS)
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_gqa_fwd_bf16(H, Hkv, D, causal):
    for i, N in enumerate([1, 17, 129, 300]):
        dev, ref = prepare("bf16", (2, H, N, D), 3000 + 17 * i + H + Hkv + D, hkv=Hkv)
        scale = 1.0 / math.sqrt(D)
        o, lse = fa.fwd(dev["q"], dev["k"], dev["v"], causal=causal, scale=scale)
        o_ref, lse_ref = attention.forward(ref["q"], ref["k"], ref["v"], causal, scale)
        eo, el = max_abs(to_f64(o), o_ref), max_abs(to_f64(lse), lse_ref)
        print(f"[gqa fwd H{H}/{Hkv} D{D} N{N} causal={causal}] O {eo:.3e} lse {el:.3e}", flush=True)
        assert eo <= TOL_BF16_O and el <= TOL_BF16_LSE


@pytest.mark.parametrize("causal", [False, True])
def test_gqa_fwd_f32(causal):
    dev, ref = prepare("f32", (1, 4, 200, 64), 3100, hkv=2)
    o, lse = fa.fwd(dev["q"], dev["k"], dev["v"], causal=causal, scale=0.125)
    o_ref, lse_ref = attention.forward(ref["q"], ref["k"], ref["v"], causal, 0.125)
    assert max_abs(to_f64(o), o_ref) <= TOL_F32 and max_abs(to_f64(lse), lse_ref) <= TOL_F32


def test_gqa_fwd_equals_copied_heads():
    """Sharing K/V heads gives bitwise the outputs of giving every query head its own copy."""
    dev, _ = prepare("bf16", (2, 8, 333, 128), 3200, hkv=2)
    for causal in (False, True):
        o, lse = fa.fwd(dev["q"], dev["k"], dev["v"], causal=causal)
        kr = dev["k"].repeat_interleave(4, dim=1).contiguous()
        vr = dev["v"].repeat_interleave(4, dim=1).contiguous()
        o_r, lse_r = fa.fwd(dev["q"], kr, vr, causal=causal)
        torch.cuda.synchronize()
        assert torch.equal(o, o_r) and torch.equal(lse, lse_r)


def _check_grads(g, g_ref, tag, group):
    """dQ at the bf16 gradient bound; dK and dV, each a sum of `group` per-head contributions with
    independent bf16 operand rounding, at that bound times sqrt(group)."""
    errs = [grad_err(a, b) for a, b in zip(g, g_ref)]
    rels = [rel_fro(a, b) for a, b in zip(g, g_ref)]
    tols = [TOL_BF16_GRAD, TOL_BF16_GRAD * math.sqrt(group), TOL_BF16_GRAD * math.sqrt(group)]
    print(f"[{tag}] max(|d|-ulp) dQ={errs[0]:.3e} dK={errs[1]:.3e} dV={errs[2]:.3e} rel={max(rels):.3e}", flush=True)
    assert all(e <= t for e, t in zip(errs, tols)), (tag, errs, tols)
    if g[0].shape[2] >= 64:
        assert max(rels) <= 2e-2, (tag, rels)


@pytest.mark.parametrize("variant", sorted(VARIANTS))
@pytest.mark.parametrize("H,Hkv", GROUPS)
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_gqa_bwd(variant, H, Hkv, D, causal):
    for i, N in enumerate([1, 33, 130, 257]):
        dev, ref = prepare("bf16", (1, H, N, D), 3300 + 13 * i + H + Hkv + D, with_grad=True, hkv=Hkv)
        scale = 1.0 / math.sqrt(D)
        o, lse = fa.fwd(dev["q"], dev["k"], dev["v"], causal=causal, scale=scale)
        g = fa.bwd(dev["q"], dev["k"], dev["v"], o, dev["do"], lse, causal=causal, scale=scale,
                   variant=VARIANTS[variant])
        torch.cuda.synchronize()
        assert g[1].shape == dev["k"].shape and g[2].shape == dev["v"].shape
        g_ref = attention.backward(ref["q"], ref["k"], ref["v"], ref["do"], causal, scale)
        _check_grads([to_f64(x) for x in g], g_ref, f"gqa bwd {variant} H{H}/{Hkv} D{D} N{N} causal={causal}",
                     H // Hkv)


def test_gqa_bwd_deterministic_is_bitwise_stable():
    dev, _ = prepare("bf16", (2, 8, 400, 128), 3400, with_grad=True, hkv=2)
    o, lse = fa.fwd(dev["q"], dev["k"], dev["v"], causal=True)
    ref = fa.bwd(dev["q"], dev["k"], dev["v"], o, dev["do"], lse, causal=True, variant=fa.FA_BWD_DETERMINISTIC)
    for _ in range(3):
        g = fa.bwd(dev["q"], dev["k"], dev["v"], o, dev["do"], lse, causal=True, variant=fa.FA_BWD_DETERMINISTIC)
        for a, b in zip(g, ref):
            assert torch.equal(a, b)


def test_gqa_workload_fwd_sampled_rows():
    """B=4 H=32 (8 K/V heads) N=2048 D=128 bf16 causal at full size, the launch bench.py times; sampled rows."""
    w = inputs.WORKLOADS["gqa_causal_bf16"]
    dev, ref = prepare("bf16", w.shape, w.seed, hkv=w.hkv)
    o, lse = fa.fwd(dev["q"], dev["k"], dev["v"], causal=w.causal)
    torch.cuda.synchronize()
    rows = sample_rows(w.N)
    o_ref, lse_ref = attention.forward(ref["q"], ref["k"], ref["v"], w.causal, w.scale, rows=rows)
    og, lg = to_f64(o)[:, :, rows], to_f64(lse)[:, :, rows]
    eo, el, rf = max_abs(og, o_ref), max_abs(lg, lse_ref), rel_fro(og, o_ref)
    print(f"[{w.name} fwd] O {eo:.3e} lse {el:.3e} rel {rf:.3e}", flush=True)
    assert eo <= TOL_BF16_O and el <= TOL_BF16_LSE and rf <= REL_BF16


def test_gqa_workload_bwd_two_groups():
    """Full-size backward; every element of two K/V-head groups (their 4 query heads each) against the oracle."""
    w = inputs.WORKLOADS["gqa_causal_bf16"]
    dev, ref = prepare("bf16", w.shape, w.seed, with_grad=True, hkv=w.hkv)
    o, lse = fa.fwd(dev["q"], dev["k"], dev["v"], causal=w.causal)
    g = fa.bwd(dev["q"], dev["k"], dev["v"], o, dev["do"], lse, causal=w.causal, variant=fa.FA_BWD_DETERMINISTIC)
    torch.cuda.synchronize()
    G = w.H // w.hkv
    for b, kh in ((0, 0), (3, 5)):
        qs = slice(kh * G, (kh + 1) * G)
        g_ref = attention.backward(ref["q"][b:b + 1, qs], ref["k"][b:b + 1, kh:kh + 1], ref["v"][b:b + 1, kh:kh + 1],
                                   ref["do"][b:b + 1, qs], w.causal, w.scale)
        mine = [to_f64(g[0][b:b + 1, qs]), to_f64(g[1][b:b + 1, kh:kh + 1]), to_f64(g[2][b:b + 1, kh:kh + 1])]
        _check_grads(mine, g_ref, f"{w.name} bwd b{b} kv{kh}", G)


def test_gqa_long_causal_forward_sampled_rows():
    """B=1 H=32 (8 K/V heads) N=32768 D=64 bf16 causal: 256 query tiles per head, so the launch takes the
    order of long causal forwards (each XCD runs its K/V groups one after another, the four query heads of a
    group together); sampled rows of every head."""
    N = 32768
    dev, ref = prepare("bf16", (1, 32, N, 64), 9100, hkv=8)
    o, lse = fa.fwd(dev["q"], dev["k"], dev["v"], causal=True)
    torch.cuda.synchronize()
    rows = sample_rows(N)
    o_ref, lse_ref = attention.forward(ref["q"], ref["k"], ref["v"], True, 1.0 / 8.0, rows=rows)
    og, lg = to_f64(o)[:, :, rows], to_f64(lse)[:, :, rows]
    eo, el, rf = max_abs(og, o_ref), max_abs(lg, lse_ref), rel_fro(og, o_ref)
    print(f"[gqa long fwd H32/8 N{N} D64] O {eo:.3e} lse {el:.3e} rel {rf:.3e}", flush=True)
    assert eo <= TOL_BF16_O and el <= TOL_BF16_LSE and rf <= REL_BF16
