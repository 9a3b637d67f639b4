"""GPU parity of block-sparse attention (fa_block_lists, fa_fwd_sparse, fa_bwd_sparse).

The block lists are integer work and are compared exactly with a CPU construction from the mask and
the causal / window band. Outputs are compared with the oracle's block_mask definition; an all-true
mask must reproduce the dense call, and rows whose blocks are all dropped give O = 0, lse = -inf.
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
BLK = fa.BLOCK


def _win(w):
    return -1 if w is None else w


def _mask(B, H, Nq, Nk, density, seed):
    nqb, nkb = -(-Nq // BLK), -(-Nk // BLK)
    return np.random.default_rng(seed).random((B, H, nqb, nkb)) < density


def _expected_lists(m, Nq, Nk, causal, w):
    """Listed blocks by the band rule: mask set, first key <= key_hi(last row), last key >= key_lo(first row)."""
    B, H, nqb, nkb = m.shape
    off = Nk - Nq

    def hi(i):
        return min(Nk - 1, i + off) if causal else Nk - 1

    def lo(i):
        return max(0, i + off - w) if w >= 0 else 0

    live = np.zeros_like(m)
    for qb in range(nqb):
        i0, i1 = qb * BLK, min(qb * BLK + BLK, Nq) - 1
        for kb in range(nkb):
            j0, j1 = kb * BLK, min(kb * BLK + BLK, Nk) - 1
            live[:, :, qb, kb] = m[:, :, qb, kb] & (j0 <= hi(i1)) & (j1 >= lo(i0)) & (lo(i1) <= hi(i1))
    return live


@pytest.mark.parametrize("Nq,Nk,causal,window", [(1000, 1000, True, None), (300, 1200, True, None),
                                                 (700, 513, False, None), (1024, 1024, True, 200)])
def test_block_lists_exact(Nq, Nk, causal, window):
    B, H = 2, 3
    m = _mask(B, H, Nq, Nk, 0.6, 7000 + Nq)
    bl = fa.block_lists(torch.from_numpy(m).to(DEV), Nq, Nk, causal, window)
    torch.cuda.synchronize()
    live = _expected_lists(m, Nq, Nk, causal, _win(window))
    kv_count, kv_index = bl.kv_count.cpu().numpy(), bl.kv_index.cpu().numpy()
    q_count, q_index = bl.q_count.cpu().numpy(), bl.q_index.cpu().numpy()
    for b in range(B):
        for h in range(H):
            for qb in range(live.shape[2]):
                want = np.nonzero(live[b, h, qb])[0]
                assert kv_count[b, h, qb] == len(want) and np.array_equal(kv_index[b, h, qb, :len(want)], want)
            for kb in range(live.shape[3]):
                want = np.nonzero(live[b, h, :, kb])[0]
                assert q_count[b, h, kb] == len(want) and np.array_equal(q_index[b, h, kb, :len(want)], want)


def test_block_lists_broadcast_mask():
    """A mask broadcast over batch and heads (zero strides) lists the same blocks for every head."""
    Nq = Nk = 900
    m = _mask(1, 1, Nq, Nk, 0.5, 7100)
    mt = torch.from_numpy(m).to(DEV).expand(2, 4, -1, -1)
    bl = fa.block_lists(mt, Nq, Nk, True)
    torch.cuda.synchronize()
    live = _expected_lists(np.broadcast_to(m, (2, 4) + m.shape[2:]), Nq, Nk, True, -1)
    assert np.array_equal(bl.kv_count.cpu().numpy(), live.sum(axis=3))
    assert np.array_equal(bl.q_count.cpu().numpy(), live.sum(axis=2))


# (dtype, B, H, Hkv, Nq, Nk, D, causal, window, density)
FWD_CASES = [("bf16", 2, 4, 4, 1000, 1000, 128, True, None, 0.5), ("bf16", 1, 4, 2, 640, 1300, 64, True, None, 0.4),
             ("bf16", 1, 2, 2, 520, 700, 256, False, None, 0.6), ("bf16", 2, 4, 2, 1024, 1024, 128, True, 300, 0.7),
             ("f32", 1, 2, 1, 400, 400, 64, True, None, 0.5), ("f32", 1, 2, 2, 300, 520, 128, False, 100, 0.6)]


@pytest.mark.parametrize("case", FWD_CASES, ids=lambda c: "-".join(map(str, c)))
def test_sparse_fwd(case):
    dt, B, H, Hkv, Nq, Nk, D, causal, window, dens = case
    dev, ref = prepare(dt, (B, H, Nq, D), 7200 + Nq + Nk + D, hkv=Hkv, nk=Nk)
    m = _mask(B, H, Nq, Nk, dens, 7300 + Nq)
    m[0, 0, 1, :] = False  # a query block whose rows keep no key
    bl = fa.block_lists(torch.from_numpy(m).to(DEV), Nq, Nk, causal, window)
    o, lse = fa.fwd(dev["q"], dev["k"], dev["v"], causal=causal, window=window, block_lists=bl)
    torch.cuda.synchronize()
    o_ref, lse_ref = attention.forward(ref["q"], ref["k"], ref["v"], causal, 1 / math.sqrt(D), window=_win(window),
                                       block_mask=m)
    og, lg = to_f64(o), to_f64(lse)
    empty = lse_ref == -np.inf
    assert empty[0, 0, BLK:2 * BLK].all()
    assert np.all(lg[empty] == -np.inf) and np.all(og[empty] == 0.0)
    eo, el = max_abs(og, o_ref), max_abs(lg[~empty], lse_ref[~empty])
    print(f"[sparse fwd {case}] O {eo:.3e} lse {el:.3e}", flush=True)
    tol_o, tol_l = (TOL_F32, TOL_F32) if dt == "f32" else (TOL_BF16_O, TOL_BF16_LSE)
    assert eo <= tol_o and el <= tol_l


@pytest.mark.parametrize("variant", sorted(VARIANTS))
@pytest.mark.parametrize("case", [(2, 4, 4, 1000, 1000, 128, True, None, 0.5), (1, 4, 2, 640, 1300, 64, True, None, 0.4),
                                  (1, 4, 2, 700, 520, 128, False, None, 0.6), (1, 4, 4, 1024, 1024, 64, True, 300, 0.7)],
                         ids=lambda c: "-".join(map(str, c)))
def test_sparse_bwd(variant, case):
    B, H, Hkv, Nq, Nk, D, causal, window, dens = case
    dev, ref = prepare("bf16", (B, H, Nq, D), 7400 + Nq + Nk + D, with_grad=True, hkv=Hkv, nk=Nk)
    m = _mask(B, H, Nq, Nk, dens, 7500 + Nq)
    m[0, 0, 1, :] = False
    bl = fa.block_lists(torch.from_numpy(m).to(DEV), Nq, Nk, causal, window)
    o, lse = fa.fwd(dev["q"], dev["k"], dev["v"], causal=causal, window=window, block_lists=bl)
    g = fa.bwd(dev["q"], dev["k"], dev["v"], o, dev["do"], lse, causal=causal, window=window,
               variant=VARIANTS[variant], block_lists=bl)
    torch.cuda.synchronize()
    g_ref = attention.backward(ref["q"], ref["k"], ref["v"], ref["do"], causal, 1 / math.sqrt(D),
                               window=_win(window), block_mask=m)
    errs = [grad_err(to_f64(a), b) for a, b in zip(g, g_ref)]
    rels = [rel_fro(to_f64(a), b) for a, b in zip(g, g_ref)]
    print(f"[sparse bwd {variant} {case}] dQ {errs[0]:.3e} dK {errs[1]:.3e} dV {errs[2]:.3e} rel {max(rels):.3e}",
          flush=True)
    g2 = TOL_BF16_GRAD * math.sqrt(H // Hkv)
    assert errs[0] <= TOL_BF16_GRAD and errs[1] <= g2 and errs[2] <= g2 and max(rels) <= 2e-2
    assert not g[0][0, 0, BLK:2 * BLK].any(), "rows whose blocks are all dropped must get dQ = 0"


@pytest.mark.parametrize("causal", [False, True])
def test_all_true_mask_equals_dense(causal):
    """Every block kept: the same tiles as the dense call (plus fully masked ones past the last key),
    so the same values (as numbers; a zero may change sign)."""
    B, H, Nq, Nk, D = 2, 4, 777, 777, 128
    dev, _ = prepare("bf16", (B, H, Nq, D), 7600, with_grad=True)
    m = np.ones((B, H, -(-Nq // BLK), -(-Nk // BLK)), dtype=bool)
    bl = fa.block_lists(torch.from_numpy(m).to(DEV), Nq, Nk, causal)
    o, lse = fa.fwd(dev["q"], dev["k"], dev["v"], causal=causal, block_lists=bl)
    o_d, lse_d = fa.fwd(dev["q"], dev["k"], dev["v"], causal=causal)
    g = fa.bwd(dev["q"], dev["k"], dev["v"], o, dev["do"], lse, causal=causal, variant=fa.FA_BWD_DETERMINISTIC,
               block_lists=bl)
    g_d = fa.bwd(dev["q"], dev["k"], dev["v"], o_d, dev["do"], lse_d, causal=causal,
                 variant=fa.FA_BWD_DETERMINISTIC)
    torch.cuda.synchronize()
    assert torch.equal(o, o_d) and torch.equal(lse, lse_d)
    assert all(torch.equal(a, b) for a, b in zip(g, g_d))


@pytest.mark.parametrize("D,window", [(64, -1), (128, -1), (256, -1), (128, 200)])
def test_sparse_fp8_forward_runs_the_listed_blocks(D, window):
    """The fp8 forward takes the same lists (and a window): with unit descales it matches the oracle on decoded
    codes."""
    from oracle import codecs
    B, H, N = 1, 2, 640
    rng = np.random.default_rng(7700 + D)
    codes = [codecs.f64_to_e4m3(rng.standard_normal((B, H, N, D))) for _ in range(3)]
    qd, kd, vd = (torch.from_numpy(c).to(DEV) for c in codes)
    m = _mask(B, H, N, N, 0.5, 7701)
    bl = fa.block_lists(torch.from_numpy(m).to(DEV), N, N, True, None if window < 0 else window)
    o = torch.empty((B, H, N, D), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=DEV)
    L = fa.lib()
    fa._check(L.fa_fwd_sparse(qd.data_ptr(), kd.data_ptr(), vd.data_ptr(), o.data_ptr(), lse.data_ptr(), B, H, H, N,
                              N, D, 1, window, 1 / math.sqrt(D), fa.FA_FP8_E4M3, bl.kv_count.data_ptr(),
                              bl.kv_index.data_ptr(), None))
    torch.cuda.synchronize()
    vals = [codecs.e4m3_to_f64(c) for c in codes]
    o_ref, lse_ref = attention.forward(vals[0], vals[1], vals[2], True, 1 / math.sqrt(D), window=window,
                                       block_mask=m)
    live = lse_ref != -np.inf
    assert np.all(to_f64(lse)[~live] == -np.inf) and np.all(to_f64(o)[~live] == 0)
    assert max_abs(to_f64(o), o_ref) <= 6e-2 and max_abs(to_f64(lse)[live], lse_ref[live]) <= 6e-2


def test_workload_sparse_bf16():
    """The block-sparse workload (B2 H16 N8192 D128 causal, banded + global + strided blocks) at full size,
    as the bench launches it: sampled forward rows of two heads and every gradient element of one head."""
    from tiled_online_softmax_amd import inputs
    from gpu_util import sample_rows
    w = inputs.WORKLOADS["sparse_bf16"]
    dev, ref = prepare("bf16", w.shape, w.seed, with_grad=True)
    m = w.block_mask()
    bl = fa.block_lists(torch.from_numpy(m).to(DEV).expand(w.B, w.H, -1, -1), w.N, w.N, True)
    o, lse = fa.fwd(dev["q"], dev["k"], dev["v"], causal=True, block_lists=bl)
    g = fa.bwd(dev["q"], dev["k"], dev["v"], o, dev["do"], lse, causal=True, variant=fa.FA_BWD_DETERMINISTIC,
               block_lists=bl)
    torch.cuda.synchronize()
    rows = sample_rows(w.N)
    for b, h in ((0, 0), (1, 15)):
        sl = (slice(b, b + 1), slice(h, h + 1))
        o_ref, lse_ref = attention.forward(ref["q"][sl], ref["k"][sl], ref["v"][sl], True, w.scale, rows=rows,
                                           block_mask=m)
        eo = max_abs(to_f64(o)[sl][:, :, rows], o_ref)
        el = max_abs(to_f64(lse)[sl][:, :, rows], lse_ref)
        print(f"[sparse workload fwd b{b} h{h}] O {eo:.3e} lse {el:.3e}", flush=True)
        assert eo <= TOL_BF16_O and el <= TOL_BF16_LSE
    sl = (slice(1, 2), slice(7, 8))
    g_ref = attention.backward(ref["q"][sl], ref["k"][sl], ref["v"][sl], ref["do"][sl], True, w.scale, block_mask=m)
    errs = [grad_err(to_f64(a)[sl], r) for a, r in zip(g, g_ref)]
    print(f"[sparse workload bwd] dQ {errs[0]:.3e} dK {errs[1]:.3e} dV {errs[2]:.3e}", flush=True)
    assert max(errs) <= TOL_BF16_GRAD
