"""Helpers for the GPU parity tests: move seeded inputs to the device and compare to the oracle."""
from __future__ import annotations

import numpy as np
import torch

from oracle import codecs
from tiled_online_softmax_amd import inputs

DEV = "cuda:0"

# Max-abs tolerances (float32 path, bf16 forward O / lse, bf16 backward, fp8 forward).
TOL_F32 = 1e-5
TOL_BF16_O, TOL_BF16_LSE = 2e-2, 1e-2
TOL_BF16_GRAD = 2e-2
TOL_FP8 = 6e-2
# Relative Frobenius diagnostics that catch near-uniform outputs an absolute bound would miss.
REL_BF16, REL_FP8 = 1e-2, 5e-2


def bf16_tensor(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(DEV)


def f32_tensor(x: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(DEV)


def to_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu", torch.float64).numpy()


def prepare(dtype: str, shape, seed: int, multiplier: float = 1.0, with_grad: bool = False, hkv=None, nk=None,
            kv_shape=None):
    """Draw Q, K, V (and dO) and return (device tensors dict, float64 oracle inputs dict).

    hkv, nk: K/V head count and key length when they differ from Q's (K and V get [B, hkv, nk, D]);
    kv_shape: K/V's whole shape instead (e.g. for packed [total, heads, D] tensors).
    """
    if kv_shape is None and (hkv is not None or nk is not None):
        kv_shape = (shape[0], shape[1] if hkv is None else hkv, shape[2] if nk is None else nk, shape[3])
    arrs = inputs.draw(tuple(shape), seed, 4 if with_grad else 3, multiplier, kv_shape=kv_shape)
    names = ["q", "k", "v", "do"][: len(arrs)]
    dev, ref = {}, {}
    for n, x in zip(names, arrs):
        if dtype == "f32":
            dev[n] = f32_tensor(x)
            ref[n] = x.astype(np.float64)
        elif dtype == "bf16":
            bits = inputs.f32_to_bf16_bits(x)
            dev[n] = bf16_tensor(bits)
            ref[n] = codecs.bf16_to_f64(bits)
        else:
            raise ValueError(dtype)
    return dev, ref


def max_abs(a: np.ndarray, b: np.ndarray) -> float:
    assert np.isfinite(a).all(), "non-finite GPU output"
    return float(np.max(np.abs(a - b))) if a.size else 0.0


# One bf16 rounding unit: a value stored as bf16 is off by at most half an ulp, which is at most
# 2^-8 of its magnitude (at the bottom of a binade). No bf16 output can meet a fixed max-abs bound
# below 2^-8 max|g|, and the backward's gradients reach |g| ~ 5 (2^-8 * 5 = 0.02).
BF16_ULP_REL = 2.0 ** -8


def grad_err(a: np.ndarray, ref: np.ndarray) -> float:
    """Backward error measure: max over elements of |a - ref| - 2^-8 |ref|, i.e. the error beyond one
    bf16 rounding unit of the exact gradient; compared with the max-abs gradient tolerance."""
    assert np.isfinite(a).all(), "non-finite GPU output"
    return float(np.max(np.abs(a - ref) - BF16_ULP_REL * np.abs(ref))) if a.size else 0.0


def rel_fro(a: np.ndarray, b: np.ndarray) -> float:
    den = float(np.linalg.norm(b))
    return float(np.linalg.norm(a - b)) / den if den > 0 else float(np.linalg.norm(a))


def sample_rows(N: int, head_rows: int = 512, stride: int = 61, tail: int = 512) -> np.ndarray:
    """Rows checked at full size: a prefix, every `stride`-th row, and a suffix."""
    rows = set(range(min(N, head_rows))) | set(range(0, N, stride)) | set(range(max(0, N - tail), N))
    return np.array(sorted(rows), dtype=np.int64)
