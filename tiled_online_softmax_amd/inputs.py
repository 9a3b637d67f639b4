"""Seeded synthetic inputs shared by the tests, the smoke check and the bench.

This module draws random numbers and encodes them as the storage types the
kernels read (fp32, or bf16 bit patterns). It holds none of the attention
arithmetic and none of the FP8 quantisation recipe: those live, separately,
in the HIP library and in the oracle.

Recipe (the same everywhere):
  * generator: numpy ``default_rng(seed)`` (PCG64), ``standard_normal`` in
    float32, drawn in the order Q, K, V, dO; Q and dO have shape [B, H, N, D],
    K and V [B, Hkv, N, D] (Hkv = H except for grouped-query workloads);
  * an optional multiplier (0.5 for the large-head-dim workload) is applied
    in float32, which is exact for a power of two;
  * bf16 inputs are the round-to-nearest-even bf16 of those float32 values.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, Optional, Tuple

import numpy as np

SEED_BASE = 20261203


@dataclasses.dataclass(frozen=True)
class Workload:
    """One attention problem: shapes, storage type and masking."""

    name: str
    B: int
    H: int
    N: int
    D: int
    dtype: str  # "f32", "bf16" or "fp8" (fp8: e4m3 codes quantised from f32 draws)
    causal: bool
    passes: str  # "fwd" or "bwd"
    multiplier: float = 1.0
    seed: int = SEED_BASE
    hkv: Optional[int] = None  # K/V heads (grouped-query attention); None means H
    nk: Optional[int] = None   # key length; None means N (causal is aligned at the bottom right)
    window: Optional[int] = None  # left window; None means none
    # Packed sequences: their lengths (queries = keys within a sequence); B = len(lengths), N = max.
    lengths: Optional[Tuple[int, ...]] = None
    # Block sparsity: the name of a block-mask pattern (see block_mask).
    block_pattern: Optional[str] = None

    @property
    def scale(self) -> float:
        return 1.0 / float(np.sqrt(self.D))

    @property
    def shape(self):
        """[B, H, N, D], or [total rows, H, D] for packed sequences."""
        if self.lengths is not None:
            return (int(sum(self.lengths)), self.H, self.D)
        return (self.B, self.H, self.N, self.D)

    @property
    def kv_shape(self):
        hkv = self.H if self.hkv is None else self.hkv
        if self.lengths is not None:
            return (int(sum(self.lengths)), hkv, self.D)
        return (self.B, hkv, self.N if self.nk is None else self.nk, self.D)

    def cu_seqlens(self) -> np.ndarray:
        """int32 [B + 1] row offsets of the packed sequences."""
        return np.concatenate([[0], np.cumsum(self.lengths)]).astype(np.int32)

    def block_mask(self) -> np.ndarray:
        """Boolean [1, 1, nqb, nkb] block mask (128 x 128 blocks, the same for every head) of the pattern:
        "local_global_strided" keeps a query block's own and previous key blocks, key block 0 and every
        4th key block (a banded pattern with global and strided blocks)."""
        nqb, nkb = -(-self.N // 128), -(-(self.N if self.nk is None else self.nk) // 128)
        qb = np.arange(nqb)[:, None]
        kb = np.arange(nkb)[None, :]
        if self.block_pattern == "local_global_strided":
            m = (kb >= qb - 1) & (kb <= qb) | (kb == 0) | (kb % 4 == 0)
        else:
            raise ValueError(f"unknown block pattern {self.block_pattern!r}")
        return m[None, None]

    def pairs(self) -> float:
        """(query, key) pairs one head of one batch entry computes (the mean over entries for packed
        sequences): N^2, halved for causal with equal lengths, no window and no block mask; otherwise the
        exact count of kept pairs."""
        if self.lengths is not None:
            n = np.asarray(self.lengths, dtype=np.float64)
            return float((n * (n + 1) / 2 if self.causal else n * n).sum() / len(n))
        nk = self.N if self.nk is None else self.nk
        if self.block_pattern is not None:
            i = np.arange(self.N, dtype=np.int64)[:, None]
            j = np.arange(nk, dtype=np.int64)[None, :]
            keep = self.block_mask()[0, 0][i // 128, j // 128]
            if self.causal:
                keep &= j <= i + nk - self.N
            if self.window is not None:
                keep &= j >= i + nk - self.N - self.window
            return float(keep.sum())
        if self.window is None and (not self.causal or nk == self.N):
            return self.N * nk / 2.0 if self.causal else float(self.N * nk)
        i = np.arange(self.N, dtype=np.int64)
        off = nk - self.N
        lo = np.maximum(0, i + off - self.window) if self.window is not None else np.zeros_like(i)
        hi = np.minimum(nk - 1, i + off) if self.causal else np.full_like(i, nk - 1)
        return float(np.maximum(0, hi - lo + 1).sum())

    def fwd_flops(self) -> float:
        """Two contractions (QK^T and PV) over the kept pairs, D multiply-adds each, 2 flops per FMA."""
        return 4.0 * self.B * self.H * self.pairs() * self.D

    def bwd_flops(self) -> float:
        """Five contractions (S, dV, dP, dQ, dK) over the kept pairs."""
        return 10.0 * self.B * self.H * self.pairs() * self.D


# The five workloads the library is specified and measured on.
WORKLOADS: Dict[str, Workload] = {
    "single_head_f32": Workload("single_head_f32", 1, 1, 256, 64, "f32", False, "fwd", seed=SEED_BASE + 1),
    "mh_causal_bf16": Workload("mh_causal_bf16", 4, 16, 2048, 128, "bf16", True, "fwd", seed=SEED_BASE + 2),
    "d256_bf16": Workload("d256_bf16", 1, 8, 8192, 256, "bf16", False, "fwd", multiplier=0.5, seed=SEED_BASE + 3),
    "bwd_causal_bf16": Workload("bwd_causal_bf16", 2, 16, 4096, 64, "bf16", True, "bwd", seed=SEED_BASE + 4),
    "long_fp8_causal": Workload("long_fp8_causal", 1, 32, 32768, 128, "fp8", True, "fwd", seed=SEED_BASE + 5),
    # The backward at the largest head dimension: the large-head-dim workload's shape and values, causal.
    "bwd_d256_bf16": Workload("bwd_d256_bf16", 1, 8, 8192, 256, "bf16", True, "bwd", multiplier=0.5,
                              seed=SEED_BASE + 11),
    # The e4m3 forward at the largest head dimension: causal, 16 heads of 16384 rows.
    "fp8_d256_causal": Workload("fp8_d256_causal", 1, 16, 16384, 256, "fp8", True, "fwd", seed=SEED_BASE + 12),
    # Grouped-query attention (a NEXT-row extension): 32 query heads sharing 8 K/V heads.
    "gqa_causal_bf16": Workload("gqa_causal_bf16", 4, 32, 2048, 128, "bf16", True, "fwd+bwd", seed=SEED_BASE + 6,
                                hkv=8),
    # Queries extending a cached prefix (1024 new rows after 3072 cached keys), causal at the bottom right.
    "prefill_bf16": Workload("prefill_bf16", 4, 16, 1024, 128, "bf16", True, "fwd+bwd", seed=SEED_BASE + 7, nk=4096),
    # Sliding window: every row keeps the 1024 keys ending at its diagonal.
    "swa_bf16": Workload("swa_bf16", 2, 16, 8192, 128, "bf16", True, "fwd+bwd", seed=SEED_BASE + 8, window=1023),
    # Packed batch of 16 causal sequences of mixed lengths (18,329 rows).
    "varlen_bf16": Workload("varlen_bf16", 16, 16, 4096, 128, "bf16", True, "fwd+bwd", seed=SEED_BASE + 9,
                            lengths=(4096, 3000, 2048, 2048, 1500, 1024, 1024, 1000, 800, 512, 512, 300, 256, 128,
                                     64, 17)),
    # Block-sparse causal attention: banded + global + strided 128 x 128 blocks.
    "sparse_bf16": Workload("sparse_bf16", 2, 16, 8192, 128, "bf16", True, "fwd+bwd", seed=SEED_BASE + 10,
                            block_pattern="local_global_strided"),
}


def draw(shape, seed: int, count: int = 3, multiplier: float = 1.0, kv_shape=None):
    """Return ``count`` float32 arrays (Q, K, V[, dO]) from one PCG64 stream.

    Q and dO have ``shape``; K and V have ``kv_shape`` (default ``shape``).
    """
    rng = np.random.default_rng(seed)
    shapes = [shape, kv_shape or shape, kv_shape or shape, shape][:count]
    out = []
    for shp in shapes:
        x = rng.standard_normal(size=shp, dtype=np.float32)
        if multiplier != 1.0:
            x = x * np.float32(multiplier)
        out.append(x)
    return out


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bf16 (nearest, ties to even); returns the uint16 bit patterns.

    Inputs here are finite normal draws, so no NaN handling is needed; a NaN
    input raises rather than being silently encoded.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    if not np.isfinite(x).all():
        raise ValueError("f32_to_bf16_bits: non-finite input")
    u = x.view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to float32 (exact)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def make(w: Workload, with_grad: Optional[bool] = None, seed: Optional[int] = None, shape=None, kv_shape=None):
    """Draw the inputs of workload ``w``.

    Returns a dict with float32 draws ``q, k, v`` (and ``do`` for backward
    workloads) and, for bf16 workloads, the bf16 bit patterns ``q_bits`` etc.
    ``shape`` overrides the workload's [B, H, N, D] (used for reduced-size
    parity cases that keep the same value distribution).
    """
    if with_grad is None:
        with_grad = w.passes != "fwd"
    shp = tuple(shape) if shape is not None else w.shape
    kv = tuple(kv_shape) if kv_shape is not None else (None if shape is not None else w.kv_shape)
    arrs = draw(shp, w.seed if seed is None else seed, 4 if with_grad else 3, w.multiplier, kv_shape=kv)
    names = ["q", "k", "v", "do"][: len(arrs)]
    out = dict(zip(names, arrs))
    if w.dtype == "bf16":
        for n in names:
            out[n + "_bits"] = f32_to_bf16_bits(out[n])
    elif with_grad:
        # Gradients of the low-precision paths are taken at bf16 dO.
        out["do_bits"] = f32_to_bf16_bits(out["do"])
    return out
