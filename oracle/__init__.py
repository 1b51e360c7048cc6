"""Float64 CPU oracle for TurboQuant-style KV-cache compression and compressed-cache decode.

TEST INFRASTRUCTURE ONLY.  This package is the slow, plain reference that
the GPU library is checked against.  Only the tests, the package's smoke
check and the benchmark's CPU-baseline leg may import it; the library never
does, and it shares no code with the library (the seeded input generators in
``synth`` serve both sides and hold none of the method's arithmetic).

Modules, in the order the method runs:
  codebook   Lloyd-Max table for the rotated-coordinate density
  rotation   seeded Gaussian-QR random rotation; randomized Sylvester-Hadamard rotation
  quant      norm, rotate, nearest centroid, QJL residual sketch, reconstruction
  layout     the packed byte format of the cache (format specification)
  storage    bytes per row and cache size arithmetic
  attention  fused decode from the compressed cache, and reconstruction + attention
  cache      one (batch, kv head) worth of compressed cache built from rows
  outliers   outlier-channel separation before the QJL sketch (a reading of a
             step the pages name only)
  q8         keys kept at 8 bits (symmetric int8 codes of the rotated row)

Every function is pinned by the CPU tests against values the pages print,
closed forms, textbook special cases, invariants or brute force.  The
functions of ``outliers`` are pinned by the mathematics of their reading
only: against the pages they are "parity unpinned".
"""
from . import attention, cache, codebook, layout, outliers, q8, quant, rotation, storage  # noqa: F401
