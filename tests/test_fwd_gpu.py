"""GPU parity of the forward kernels (fp32, bf16) against the float64 oracle, through the C ABI."""
import math

import numpy as np
import pytest
import torch

from gpu_util import (REL_BF16, TOL_BF16_LSE, TOL_BF16_O, TOL_F32, max_abs, prepare, rel_fro, sample_rows, to_f64)
from oracle import attention
from tiled_online_softmax_amd import fa, inputs

pytestmark = pytest.mark.gpu


def _run(dtype, shape, causal, seed, multiplier=1.0, rescale=None, rows=None):
    dev, ref = prepare(dtype, shape, seed, multiplier)
    D = shape[-1]
    scale = 1.0 / math.sqrt(D)
    o, lse = fa.fwd(dev["q"], dev["k"], dev["v"], causal=causal, scale=scale, rescale_log2=rescale)
    torch.cuda.synchronize()
    o_ref, lse_ref = attention.forward(ref["q"], ref["k"], ref["v"], causal, scale, rows=rows)
    o_gpu, lse_gpu = to_f64(o), to_f64(lse)
    if rows is not None:
        o_gpu, lse_gpu = o_gpu[:, :, rows], lse_gpu[:, :, rows]
    return o_gpu, lse_gpu, o_ref, lse_ref


def _check(dtype, o, lse, o_ref, lse_ref, tag, f32_tol=TOL_F32, bf16_o_tol=TOL_BF16_O):
    eo, el = max_abs(o, o_ref), max_abs(lse, lse_ref)
    print(f"[{tag}] max|dO|={eo:.3e} max|dlse|={el:.3e} relO={rel_fro(o, o_ref):.3e}", flush=True)
    if dtype == "f32":
        assert eo <= f32_tol and el <= f32_tol, (tag, eo, el)
    else:
        assert eo <= bf16_o_tol and el <= TOL_BF16_LSE, (tag, eo, el)
        assert rel_fro(o, o_ref) <= REL_BF16, tag


def test_single_head_f32_workload():
    """B=1 H=1 N=256 D=64 float32, non-causal: the whole output at 1e-5."""
    w = inputs.WORKLOADS["single_head_f32"]
    o, lse, o_ref, lse_ref = _run("f32", w.shape, w.causal, w.seed)
    _check("f32", o, lse, o_ref, lse_ref, w.name)


# 28..31: rows ending just short of a 32-row wave block (a stale-accumulator bug once hid there)
SMALL_N = [1, 2, 3, 15, 16, 17, 28, 29, 30, 31, 63, 65, 127, 129, 300]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("D", [64, 128, 256])
@pytest.mark.parametrize("causal", [False, True])
def test_small_shapes(dtype, D, causal):
    """Ragged N (tails inside a tile, a single row, several tiles) for every D in the table."""
    for i, N in enumerate(SMALL_N):
        o, lse, o_ref, lse_ref = _run(dtype, (1, 2, N, D), causal, 1000 + 17 * i + D)
        _check(dtype, o, lse, o_ref, lse_ref, f"{dtype} D{D} N{N} causal={causal}")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_multi_batch_head_indexing(dtype):
    """B and H > 1 with N not a multiple of the tile: each (b, h) slice must be its own problem."""
    o, lse, o_ref, lse_ref = _run(dtype, (3, 5, 200, 64), True, 77)
    _check(dtype, o, lse, o_ref, lse_ref, f"{dtype} B3 H5 N200")


def test_mh_causal_bf16_workload_full():
    """B=4 H=16 N=2048 D=128 bf16 causal, every output element."""
    w = inputs.WORKLOADS["mh_causal_bf16"]
    o, lse, o_ref, lse_ref = _run("bf16", w.shape, w.causal, w.seed)
    _check("bf16", o, lse, o_ref, lse_ref, w.name)


def test_d256_bf16_workload_sampled():
    """B=1 H=8 N=8192 D=256 bf16 x0.5 non-causal, on sampled query rows of every head."""
    w = inputs.WORKLOADS["d256_bf16"]
    rows = sample_rows(w.N)
    o, lse, o_ref, lse_ref = _run("bf16", w.shape, w.causal, w.seed, w.multiplier, rows=rows)
    _check("bf16", o, lse, o_ref, lse_ref, w.name)
    # lse sits near ln N for these nearly uniform rows
    assert abs(float(np.mean(lse)) - math.log(w.N)) < 0.1


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("D", [64, 128, 256])
@pytest.mark.parametrize("tau", [0.0, 3.0, 8.0, 30.0])
def test_rescale_threshold_variants(tau, D, dtype):
    """Conditional rescaling is exact for every threshold: on N(0,1) inputs all thresholds meet the
    stated tolerances. Causal N = 700 spans 11 (64-key) or 22 (32-key) key tiles, so the running max
    of a row grows across tiles and tau = 0 and 3 rescale non-zero accumulators. bf16 D = 128 runs
    the phase-alternating kernel, D = 64 and 256 the software-pipelined one."""
    o, lse, o_ref, lse_ref = _run(dtype, (1, 2, 700, D), True, 5 + D, rescale=tau)
    _check(dtype, o, lse, o_ref, lse_ref, f"{dtype} D{D} tau={tau}")


# Planted keys: rows 600, 601, 650 and 1100 of K set to 6 in every coordinate. Their score for
# query i is 6 * sum_d q_id / sqrt(D) = 6 z_i with z_i ~ N(0, 1), so for about a tenth of the
# rows the score jumps far above everything seen in the first nine 64-key tiles.
PLANTED = (600, 601, 650, 1100)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("D", [64, 128, 256])
def test_rescale_on_planted_keys_default_threshold(dtype, D):
    """At the default threshold (8 in log2 units) the reference max moves, and the accumulator is
    rescaled, only when a later tile beats it by a factor 256; planted keys in late tiles force that
    on many rows of every wave. Checked at the stated tolerances."""
    N = 1200
    scale = 1.0 / math.sqrt(D)
    dev, ref = prepare(dtype, (1, 2, N, D), 6100 + D)
    for j in PLANTED:
        dev["k"][:, :, j] = 6.0
        ref["k"][:, :, j] = 6.0
    # rows whose planted score exceeds every score of the keys before the first planted one by more
    # than 8 log2 units: the reference max never exceeds those scores, so these rows must rescale
    j0 = PLANTED[0]
    s_before = np.einsum("bhid,bhjd->bhij", ref["q"], ref["k"][:, :, :j0]) * scale
    before_max = np.where(np.arange(j0)[None, :] <= np.arange(N)[:, None], s_before, -np.inf).max(axis=-1)
    planted = 6.0 * ref["q"].sum(axis=-1) * scale
    jumps = (planted - before_max) * math.log2(math.e) > 8.0
    jumps[:, :, :j0] = False  # rows before the first planted key never see one
    assert jumps.sum() >= 50, int(jumps.sum())
    o, lse = fa.fwd(dev["q"], dev["k"], dev["v"], causal=True, scale=scale)
    torch.cuda.synchronize()
    o_ref, lse_ref = attention.forward(ref["q"], ref["k"], ref["v"], True, scale)
    tag = f"{dtype} D{D} planted ({int(jumps.sum())} rows jump)"
    if dtype == "bf16":
        _check(dtype, to_f64(o), to_f64(lse), o_ref, lse_ref, tag)
        return
    # float32: O at the stated 1e-5. The stated 1e-5 on lse is for N(0,1) inputs, whose scores stay
    # below about 5; planted rows reach |s| ~ 14. A float32 score summed over D products carries a
    # rounding error of about sqrt(D) u |s| (u = 2^-24), and lse = max + ln(sum) inherits it from the
    # row's dominant scores, so a row's lse is held to max(1e-5, 4 sqrt(D) u max_j |s_ij|).
    s_all = np.einsum("bhid,bhjd->bhij", ref["q"], ref["k"]) * scale
    s_abs = np.where(np.arange(N)[None, :] <= np.arange(N)[:, None], np.abs(s_all), 0.0).max(axis=-1)
    tol_lse = np.maximum(TOL_F32, 4.0 * math.sqrt(D) * 2.0 ** -24 * s_abs)
    o_g, lse_g = to_f64(o), to_f64(lse)
    eo = max_abs(o_g, o_ref)
    dl = np.abs(lse_g - lse_ref)
    print(f"[{tag}] max|dO|={eo:.3e} max|dlse|={dl.max():.3e} max(|dlse|/tol)={(dl / tol_lse).max():.3f}",
          flush=True)
    assert eo <= TOL_F32, (tag, eo)
    assert (dl <= tol_lse).all(), (tag, float((dl / tol_lse).max()))


def test_zero_query_closed_form():
    """Q = 0: O_i is the mean of V over the kept keys and lse_i = ln(count)."""
    N, D = 333, 128
    dev, ref = prepare("bf16", (1, 1, N, D), 9)
    q0 = torch.zeros_like(dev["q"])
    for causal in (False, True):
        o, lse = fa.fwd(q0, dev["k"], dev["v"], causal=causal)
        torch.cuda.synchronize()
        cnt = np.arange(1, N + 1) if causal else np.full(N, N)
        mean_v = (np.cumsum(ref["v"][0, 0], axis=0) / cnt[:, None]) if causal else \
            np.broadcast_to(ref["v"][0, 0].mean(axis=0), (N, D))
        assert max_abs(to_f64(o)[0, 0], mean_v) <= TOL_BF16_O
        assert max_abs(to_f64(lse)[0, 0], np.log(cnt)) <= 1e-5


def test_permutation_invariance():
    """Non-causal: permuting K and V rows together leaves O and lse unchanged (tile-order independence)."""
    dev, _ = prepare("f32", (1, 2, 500, 64), 10)
    perm = torch.from_numpy(np.random.default_rng(3).permutation(500)).to(dev["q"].device)
    o1, l1 = fa.fwd(dev["q"], dev["k"], dev["v"])
    o2, l2 = fa.fwd(dev["q"], dev["k"][:, :, perm].contiguous(), dev["v"][:, :, perm].contiguous())
    torch.cuda.synchronize()
    assert max_abs(to_f64(o1), to_f64(o2)) <= 1e-5
    assert max_abs(to_f64(l1), to_f64(l2)) <= 1e-5


def test_key_shift_invariance():
    """K -> K + u shifts lse_i by scale*q_i.u and leaves O unchanged (the running max must follow)."""
    dev, ref = prepare("f32", (1, 1, 400, 64), 11)
    u = torch.full((64,), 0.75, device=dev["q"].device)
    scale = 0.125
    o1, l1 = fa.fwd(dev["q"], dev["k"], dev["v"], causal=True, scale=scale)
    o2, l2 = fa.fwd(dev["q"], (dev["k"] + u).contiguous(), dev["v"], causal=True, scale=scale)
    torch.cuda.synchronize()
    shift = scale * (ref["q"][0, 0] @ np.full(64, 0.75))
    assert max_abs(to_f64(o1), to_f64(o2)) <= 2e-5
    assert max_abs(to_f64(l2)[0, 0] - to_f64(l1)[0, 0], shift) <= 2e-5


def test_forward_is_deterministic():
    """Ten runs give bitwise-identical outputs (an LDS double-buffer race would show here)."""
    dev, _ = prepare("bf16", (2, 4, 1000, 128), 12)
    o0, l0 = fa.fwd(dev["q"], dev["k"], dev["v"], causal=True)
    for _ in range(9):
        o, l = fa.fwd(dev["q"], dev["k"], dev["v"], causal=True)
        assert torch.equal(o, o0) and torch.equal(l, l0)


# The bf16 D=128 forward has two kernels. The phase-alternating one (eight waves, 256-row query
# tiles) takes one query head per K/V head without a window, packed sequences or block lists; the
# 128-row-tile one takes everything else. Both do the same arithmetic in the same order per row.
PP_N = [1, 31, 64, 255, 256, 257, 511, 600, 1025]


@pytest.mark.parametrize("causal", [False, True])
def test_bf16_d128_kernels_agree_bitwise(causal):
    """Plain call (phase-alternating kernel) and all-true block list (128-row-tile kernel, which walks
    the same key tiles plus fully masked ones) give identical O and lse over ragged lengths."""
    for i, N in enumerate(PP_N):
        dev, _ = prepare("bf16", (1, 3, N, 128), 7900 + i)
        nb = -(-N // fa.BLOCK)
        bl = fa.block_lists(torch.ones((1, 3, nb, nb), dtype=torch.bool, device=dev["q"].device), N, N, causal)
        o_s, l_s = fa.fwd(dev["q"], dev["k"], dev["v"], causal=causal, block_lists=bl)
        o_d, l_d = fa.fwd(dev["q"], dev["k"], dev["v"], causal=causal)
        torch.cuda.synchronize()
        assert torch.equal(o_d, o_s) and torch.equal(l_d, l_s), (N, causal)


@pytest.mark.parametrize("nq,nk", [(300, 1000), (1000, 300), (257, 1)])
def test_bf16_d128_unequal_lengths_oracle(nq, nk):
    """N_q != N_k (bottom-right causal and full) on the phase-alternating kernel against the oracle."""
    for causal in (False, True):
        dev, ref = prepare("bf16", (2, 2, nq, 128), 7950 + nq + nk, nk=nk)
        o, lse = fa.fwd(dev["q"], dev["k"], dev["v"], causal=causal)
        torch.cuda.synchronize()
        o_ref, lse_ref = attention.forward(ref["q"], ref["k"], ref["v"], causal, 1.0 / math.sqrt(128))
        o_gpu, lse_gpu = to_f64(o), to_f64(lse)
        if causal and nk < nq:
            # rows before the shifted diagonal keep no key: O = 0, lse = -inf in both
            keep = np.isfinite(lse_ref)
            assert np.array_equal(keep, np.isfinite(lse_gpu))
            lse_gpu, lse_ref = np.where(keep, lse_gpu, 0.0), np.where(keep, lse_ref, 0.0)
        _check("bf16", o_gpu, lse_gpu, o_ref, lse_ref, f"Nq{nq} Nk{nk} causal={causal}")


def test_bf16_d128_k_v_row_spacings_differ():
    """K rows 512 bytes apart, V rows 256 apart (the kernel's two-offset loader) equal the contiguous call."""
    dev, _ = prepare("bf16", (2, 3, 700, 128), 7990)
    wide = torch.zeros((2, 3, 700, 256), dtype=torch.bfloat16, device=dev["q"].device)
    wide[..., :128] = dev["k"]
    k_view = wide[..., :128]
    assert k_view.stride(2) == 256 and not k_view.is_contiguous()
    for causal in (False, True):
        o_v, l_v = fa.fwd(dev["q"], k_view, dev["v"], causal=causal)
        o_c, l_c = fa.fwd(dev["q"], dev["k"], dev["v"], causal=causal)
        torch.cuda.synchronize()
        assert torch.equal(o_v, o_c) and torch.equal(l_v, l_c), causal
