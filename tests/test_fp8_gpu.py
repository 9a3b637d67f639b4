"""GPU parity of the FP8 path: per-tensor quantisation (bit-exact) and the e4m3 forward (6e-2)."""
import math

import numpy as np
import pytest
import torch

from gpu_util import DEV, REL_FP8, TOL_FP8, f32_tensor, max_abs, rel_fro, sample_rows, to_f64
from oracle import attention, codecs
from tiled_online_softmax_amd import fa, inputs

pytestmark = pytest.mark.gpu


def _quantize_both(x: np.ndarray):
    codes_gpu, desc_gpu = fa.quantize_fp8(f32_tensor(x))
    torch.cuda.synchronize()
    codes_ref, desc_ref = codecs.quantize_per_tensor(x)
    return codes_gpu, desc_gpu, codes_ref, desc_ref


@pytest.mark.parametrize("n", [1, 3, 4, 1000, 4099, 1 << 20])
def test_quantize_bit_exact(n):
    x = np.random.default_rng(n).standard_normal(n).astype(np.float32) * 3
    codes_gpu, desc_gpu, codes_ref, desc_ref = _quantize_both(x)
    np.testing.assert_array_equal(codes_gpu.cpu().numpy(), codes_ref)
    assert desc_gpu.item() == float(desc_ref)


def test_quantize_zero_tensor():
    codes_gpu, desc_gpu, _, _ = _quantize_both(np.zeros(100, np.float32))
    assert desc_gpu.item() == 1.0 and int(codes_gpu.cpu().max()) == 0


def _fp8_case(shape, causal, seed, rows=None, heads=None):
    """Quantise seeded N(0,1) draws on the GPU, run the FP8 forward, compare with the oracle.

    The oracle quantises the same float32 draws with its own codec and runs on the
    dequantised values; the codes are also compared bit-exactly (on the checked heads).
    """
    q, k, v = inputs.draw(shape, seed, 3)
    dev = [fa.quantize_fp8(f32_tensor(x)) for x in (q, k, v)]
    D = shape[-1]
    scale = 1.0 / math.sqrt(D)
    o, lse = fa.fwd_fp8(dev[0][0], dev[1][0], dev[2][0], causal=causal, scale=scale,
                        q_descale=dev[0][1], k_descale=dev[1][1], v_descale=dev[2][1])
    torch.cuda.synchronize()
    heads = list(range(shape[1])) if heads is None else heads
    ref_in = []
    for x, (codes_gpu, desc_gpu) in zip((q, k, v), dev):
        amax = np.float32(np.max(np.abs(x)))
        assert desc_gpu.item() == float(np.float32(amax / np.float32(448)))
        xs = (x[:, heads] * (np.float32(448) / amax)).astype(np.float32)
        codes_ref = codecs.f64_to_e4m3(xs.astype(np.float64))
        np.testing.assert_array_equal(codes_gpu[:, heads].cpu().numpy(), codes_ref)
        ref_in.append(codecs.dequantize(codes_ref, desc_gpu.item()))
    o_ref, lse_ref = attention.forward(*ref_in, causal, scale, rows=rows)
    o_gpu, lse_gpu = to_f64(o)[:, heads], to_f64(lse)[:, heads]
    if rows is not None:
        o_gpu, lse_gpu = o_gpu[:, :, rows], lse_gpu[:, :, rows]
    eo, el = max_abs(o_gpu, o_ref), max_abs(lse_gpu, lse_ref)
    print(f"[fp8 {shape} causal={causal}] max|dO|={eo:.3e} max|dlse|={el:.3e} relO={rel_fro(o_gpu, o_ref):.3e}",
          flush=True)
    assert eo <= TOL_FP8 and el <= TOL_FP8
    assert rel_fro(o_gpu, o_ref) <= REL_FP8


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_fp8_small(D, causal):
    for i, N in enumerate([1, 5, 64, 65, 200, 1000]):
        _fp8_case((1, 2, N, D), causal, 300 + i + D)


def test_fp8_long_context_workload_sampled():
    """B=1 H=32 N=32768 D=128 e4m3 causal: sampled rows of 4 of the 32 heads (plus bit-exact codes)."""
    w = inputs.WORKLOADS["long_fp8_causal"]
    _fp8_case(w.shape, w.causal, w.seed, rows=sample_rows(w.N), heads=[0, 9, 22, 31])


def test_fp8_unit_descales_via_fa_fwd():
    """fa_fwd with FA_FP8_E4M3 is the FP8 forward with all descales 1."""
    x = np.random.default_rng(4).standard_normal((1, 1, 100, 64)).astype(np.float32)
    codes = [codecs.f64_to_e4m3(x.astype(np.float64) * s) for s in (1.0, 0.5, 2.0)]
    t = [torch.from_numpy(c).to(DEV) for c in codes]
    o, lse = fa.fwd(t[0], t[1], t[2], causal=False, scale=0.125)
    torch.cuda.synchronize()
    o_ref, lse_ref = attention.forward(*[codecs.e4m3_to_f64(c) for c in codes], False, 0.125)
    assert max_abs(to_f64(o), o_ref) <= TOL_FP8 and max_abs(to_f64(lse), lse_ref) <= TOL_FP8
