"""fa_bwd_noalloc -- the backward with its workspace in the library's static device array -- against fa_bwd.

Two calls in a row on one GPU, the second on a smaller problem, so the second call runs on an array that
still holds the first call's contents. The atomics-free variant must equal fa_bwd bitwise (same kernels,
same order); the atomic variant adds dQ with float atomics in an unspecified order, so both are held to the
oracle's tolerance instead. Outputs are pre-filled with NaN, so a gradient the call failed to write shows.
"""
import math

import pytest
import torch

from gpu_util import TOL_BF16_GRAD, grad_err, prepare, to_f64
from oracle import attention
from tiled_online_softmax_amd import fa

pytestmark = pytest.mark.gpu

CASES = [((2, 4, 1000, 128), True), ((1, 2, 300, 64), False)]  # the second call is the smaller one


def _case(i, shape, causal, variant):
    dev, ref = prepare("bf16", shape, 9300 + i, with_grad=True)
    scale = 1.0 / math.sqrt(shape[-1])
    o, lse = fa.fwd(dev["q"], dev["k"], dev["v"], causal=causal, scale=scale)
    want = fa.bwd(dev["q"], dev["k"], dev["v"], o, dev["do"], lse, causal=causal, scale=scale, variant=variant)
    outs = [torch.full_like(dev["q"], float("nan")) for _ in range(3)]
    got = fa.bwd_noalloc(dev["q"], dev["k"], dev["v"], o, dev["do"], lse, causal=causal, scale=scale,
                         variant=variant, dq=outs[0], dk=outs[1], dv=outs[2])
    torch.cuda.synchronize()
    assert all(g.data_ptr() == t.data_ptr() for g, t in zip(got, outs))
    g_ref = attention.backward(ref["q"], ref["k"], ref["v"], ref["do"], causal, scale)
    errs = [grad_err(to_f64(g), r) for g, r in zip(got, g_ref)]
    print(f"[noalloc {shape} causal={causal} variant={variant}] max|d| vs oracle {errs}", flush=True)
    assert max(errs) <= TOL_BF16_GRAD
    return got, want


def test_noalloc_deterministic_equals_fa_bwd_bitwise():
    for i, (shape, causal) in enumerate(CASES):
        got, want = _case(i, shape, causal, fa.FA_BWD_DETERMINISTIC)
        for g, w, n in zip(got, want, ("dQ", "dK", "dV")):
            assert torch.equal(g, w), (shape, n)


def test_noalloc_atomic_variant():
    for i, (shape, causal) in enumerate(CASES):
        got, want = _case(10 + i, shape, causal, fa.FA_BWD_ATOMIC)
        for g, w in zip(got, want):
            assert grad_err(to_f64(g), to_f64(w)) <= TOL_BF16_GRAD


def test_noalloc_refuses_problems_beyond_the_scratch():
    """B4 H16 N2048 D128 with the atomic variant needs 68.2 MB of workspace (> 64 MiB): refused, with
    nothing launched; the atomics-free variant of the same problem (1 MiB) runs."""
    shape = (4, 16, 2048, 128)
    assert fa.bwd_workspace_size(*shape, variant=fa.FA_BWD_ATOMIC) > (64 << 20)
    q, k, v, o, do = (torch.zeros(shape, dtype=torch.bfloat16, device="cuda:0") for _ in range(5))
    lse = torch.zeros(shape[:3], dtype=torch.float32, device="cuda:0")
    with pytest.raises(fa.FAError) as ei:
        fa.bwd_noalloc(q, k, v, o, do, lse, causal=True, variant=fa.FA_BWD_ATOMIC)
    assert ei.value.status == fa.FA_ERR_WORKSPACE and "static scratch" in str(ei.value)
    dq, dk, dv = fa.bwd_noalloc(q, k, v, o, do, lse, causal=True, variant=fa.FA_BWD_DETERMINISTIC)
    torch.cuda.synchronize()
    # Q = K = V = dO = 0 and lse = 0: P = exp(0 - 0) = 1 on kept keys, dP = 0, D = 0, so every gradient is 0
    # except dV_j = sum of the P-weighted dO rows = 0.
    assert not dq.any() and not dk.any() and not dv.any()
