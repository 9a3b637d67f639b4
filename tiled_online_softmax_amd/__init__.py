"""libfa: exact FlashAttention-style attention for AMD MI355X (gfx950).

The compute path is the HIP library ``libfa.so`` built from ``csrc/`` and
declared in ``include/fa.h``; ``tiled_online_softmax_amd.fa`` is its thin
ctypes binding (argument marshalling only). ``inputs`` holds the seeded
synthetic input generator.
"""
