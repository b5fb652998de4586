"""CPU oracle for one MoE decoder layer's batch-1 verify step.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports, links or runs
anything under this directory; only the tests, the smoke check in
``__graft_entry__`` and the CPU-baseline leg of ``bench.py`` use it.

The oracle is a plain, slow, obviously-correct fp64 NumPy implementation of
what the layer computes.  Weights are bf16 or NVFP4 and the KV cache is bf16:
those are storage formats, so the only rounding the oracle applies is that of
the new keys and values to bf16 (nearest even) when they are written to the
cache.  No activation is rounded (see ``layer.py``).  ``brute.py`` is a
second, loop-only implementation of the same definition used to pin the
vectorised one on tiny shapes.  Neither shares code with the HIP path.
"""
from . import formats, layer, brute  # noqa: F401
