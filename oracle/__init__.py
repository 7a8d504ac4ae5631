"""CPU oracle for the speculative verification step — TEST INFRASTRUCTURE ONLY.

Plain, slow, fp64 implementations of what the hot path computes, written from
the source pages:

* ``oracle.mx``     — OCP MX-FP4 codec: E2M1 elements, E8M0 block scales,
                      32-element blocks, packed storage, round-to-nearest-even
                      quantizer.
* ``oracle.gemm``   — the verification GEMM Y = X · Ŵᵀ in fp64 on dequantized
                      weights.
* ``oracle.accept`` — the scalar propose–verify–correct loop: per-position
                      softmax, acceptance min(1, p/q), first-rejection stop,
                      residual resample or bonus draw by inverse CDF from
                      supplied uniforms.
* ``oracle.expect`` — closed forms used as pins (overlap mass, expected tokens
                      per cycle).
* ``oracle.tree``   — verification of a tree of drafts: siblings tried in
                      order against the running residual law, final draw
                      from the last law (the linear rule for a chain).
* ``oracle.kvcache`` — MX-FP4 KV cache codec: per-token head vectors coded in
                      32-element blocks along the head dimension, written at
                      cache slots.
* ``oracle.attention`` — verification attention over the MX-FP4 cache: every
                      query position sees the prefix and its own path among
                      the new positions (chain or tree masks), fp64.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package. The product library must never call it:
it shares no code, tables or helpers with the HIP path, and the HIP path never
falls back to it.

Every function is pinned by a CPU test against facts the pages or mathematics
fix (printed worked examples, the value grid, closed forms, brute force on tiny
inputs); none is "parity unpinned".
"""
from . import mx, gemm, accept, expect, tree, kvcache, attention  # noqa: F401
