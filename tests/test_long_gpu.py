"""The longest heads of the parity suite: a 262,144-row causal forward and a 65,536-row backward.

Long heads exercise the tile ranges, 32-bit in-head offsets and launch orders at their largest. The oracle
computes the sampled query rows exactly (rows are independent); for the backward, dQ rows and the dK / dV
rows of sampled keys in the last 4096 of the head are exact (a key's gradients need only the query rows
that keep it), and dV is also checked through an identity that holds at any size.
"""
import math

import numpy as np
import pytest
import torch

from gpu_util import (TOL_BF16_GRAD, grad_err, TOL_BF16_LSE, TOL_BF16_O, max_abs, prepare, rel_fro, to_f64)
from oracle import attention
from tiled_online_softmax_amd import fa

pytestmark = pytest.mark.gpu


def _rows(N):
    """A prefix, the edges of 64-, 128- and 256-row tiles, a stride through the middle, and a suffix."""
    r = set(range(min(N, 64))) | set(range(max(0, N - 64), N)) | set(range(0, N, 4099))
    for t in (64, 128, 256):
        for e in (t, N // 2 - N // 2 % t, N - N % t - t):
            r |= {e - 1, e} if e > 0 else set()
    return np.array(sorted(x for x in r if 0 <= x < N), dtype=np.int64)


def test_long_causal_forward_sampled():
    B, H, N, D = 1, 2, 262144, 128
    print(f"[long fwd] drawing B{B} H{H} N{N} D{D}", flush=True)
    dev, ref = prepare("bf16", (B, H, N, D), 8100)
    o, lse = fa.fwd(dev["q"], dev["k"], dev["v"], causal=True)
    torch.cuda.synchronize()
    rows = _rows(N)
    o_ref, lse_ref = attention.forward(ref["q"], ref["k"], ref["v"], True, 1.0 / math.sqrt(D), rows=rows)
    o_g, lse_g = to_f64(o)[:, :, rows], to_f64(lse)[:, :, rows]
    eo, el, rel = max_abs(o_g, o_ref), max_abs(lse_g, lse_ref), rel_fro(o_g, o_ref)
    print(f"[long fwd] {len(rows)} rows: max|dO|={eo:.3e} max|dlse|={el:.3e} relO={rel:.3e}", flush=True)
    assert eo <= TOL_BF16_O and el <= TOL_BF16_LSE and rel <= 1e-2


def _key_rows(N, span=4096):
    """Keys of the last `span` rows: a suffix, the edges of 32-, 64-, 128- and 256-key tiles, and a stride."""
    lo = N - span
    r = set(range(N - 96, N)) | set(range(lo, lo + 32)) | set(range(lo, N, 997))
    for t in (32, 64, 128, 256):
        for e in (lo + t, lo + span // 2 - (span // 2) % t, N - t):
            r |= {e - 1, e}
    return np.array(sorted(x for x in r if lo <= x < N), dtype=np.int64)


def test_long_causal_backward_dq_rows_and_dv_sum():
    B, H, N, D = 1, 2, 65536, 128
    scale = 1.0 / math.sqrt(D)
    print(f"[long bwd] drawing B{B} H{H} N{N} D{D}", flush=True)
    dev, ref = prepare("bf16", (B, H, N, D), 8200, with_grad=True)
    o, lse = fa.fwd(dev["q"], dev["k"], dev["v"], causal=True)
    dq, dk, dv = fa.bwd(dev["q"], dev["k"], dev["v"], o, dev["do"], lse, causal=True,
                        variant=fa.FA_BWD_DETERMINISTIC)
    torch.cuda.synchronize()
    rows = _rows(N)
    dq_ref = attention.backward_dq_rows(ref["q"], ref["k"], ref["v"], ref["do"], True, scale, rows)
    dq_g = to_f64(dq)[:, :, rows]
    e, rel = grad_err(dq_g, dq_ref), rel_fro(dq_g, dq_ref)
    print(f"[long bwd] {len(rows)} dQ rows: max|d|={e:.3e} rel={rel:.3e}", flush=True)
    assert e <= TOL_BF16_GRAD and rel <= 2e-2
    krows = _key_rows(N)
    dk_ref, dv_ref = attention.backward_kv_rows(ref["q"], ref["k"], ref["v"], ref["do"], True, scale, krows)
    dk_g, dv_g = to_f64(dk)[:, :, krows], to_f64(dv)[:, :, krows]
    ek, ev = grad_err(dk_g, dk_ref), grad_err(dv_g, dv_ref)
    rk, rv = rel_fro(dk_g, dk_ref), rel_fro(dv_g, dv_ref)
    print(f"[long bwd] {len(krows)} dK/dV rows: max|d| dK={ek:.3e} dV={ev:.3e} rel {rk:.3e} {rv:.3e}", flush=True)
    assert ek <= TOL_BF16_GRAD and ev <= TOL_BF16_GRAD and rk <= 2e-2 and rv <= 2e-2
    # Rows of P sum to one, so sum_j dV_j = sum_j sum_i P_ij dO_i = sum_i dO_i exactly. The GPU's dV
    # entries are bf16-rounded (relative 2^-9 each), so their sum is allowed 8 * 2^-9 * ||dV column||.
    dv64, dk64 = to_f64(dv), to_f64(dk)
    assert np.isfinite(dv64).all() and np.isfinite(dk64).all()
    lhs, rhs = dv64.sum(axis=2), ref["do"].sum(axis=2)
    bound = 8 * 2.0 ** -9 * np.sqrt((dv64 ** 2).sum(axis=2)) + 1e-3
    print(f"[long bwd] max |sum dV - sum dO| = {np.abs(lhs - rhs).max():.3e} (bound {bound.min():.3e})", flush=True)
    assert (np.abs(lhs - rhs) <= bound).all()
