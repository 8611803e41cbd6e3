"""HLWQ CPU oracle.

TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only ``tests/``, the smoke check in
``__graft_entry__.py`` and the CPU-baseline leg of ``bench.py`` may import or run
anything in this package.  The product path (``weight_quantization_amd``) never
imports it and shares no code, table or helper with it; the two meet only in the
tests, on inputs drawn by ``synth``.

Plain numpy, slow on purpose, every step written the way the model cards state
it so a reader can check it by eye:

* ``lloyd_max``: Lloyd-Max centroids and decision thresholds for N(0, 1).
* ``hlwq_ref``: block reshape, L2 norm, Walsh-Hadamard rotation, nearest
  centroid, bit packing, and their inverse, in an fp64 definition tier (D) and
  an fp32 canonical tier (C) that fixes the rounding of every intermediate.
* ``tq3_ref``: the TQ3 / scalar HIGGS variant (random-sign Walsh-Hadamard
  rotation, 8 Lloyd-Max centroids, fp32 shape-gain norm) and its SplitMix64
  sign generator, in the same two tiers.

Every function is pinned by tests in ``tests/test_oracle_*.py`` against closed
forms, textbook values, library routines or brute force.  One reading is
unpinned against the pages by necessity: the page that names TQ3's seed names no
generator, so TQ3's sign vectors (and with them bit-parity with checkpoints
made by the page's own tool) are "parity unpinned"; the generator chosen in
their place is pinned to its published outputs.
"""
from . import hlwq_ref, lloyd_max, tq3_ref  # noqa: F401
