"""Reference oracle for exact softmax attention -- TEST INFRASTRUCTURE ONLY.

A plain, slow, obviously-correct CPU implementation in float64 (numpy) of
what the HIP library computes. Only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` may import it. The HIP product
path never imports, links or calls anything here, and nothing here comes
from the HIP path: the two share only the seeded input generator, which
holds no attention arithmetic.

What it follows. The pages describe FlashAttention FA1-FA4 as orchestrations
that leave the exact attention result unchanged (page "r/mlscaling", the post
on an educational FA1-FA4 PyTorch repo, closing sentence of the version list). The
oracle is therefore that exact math written out: the full score matrix is
materialised, masked, and normalised with an ordinary softmax -- no tiling,
no online rescaling.

Modules:
  * ``attention`` -- forward (O, lse) and backward (dQ, dK, dV) in float64;
  * ``codecs``    -- bf16 widening and OCP e4m3 (E4M3FN) decode/encode, and the
                     per-tensor amax FP8 quantisation recipe;
  * ``brute``     -- pure-Python scalar loops for tiny inputs (N <= 16).

Every function is pinned in ``tests/test_oracle.py`` / ``tests/test_codecs.py``
to something other than itself (closed forms, hand-derived worked examples,
invariants, finite differences, torch's CPU float64 library routines).
"""
from . import attention, brute, codecs  # noqa: F401
