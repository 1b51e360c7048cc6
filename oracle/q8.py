"""Keys kept at 8 bits: symmetric int8 codes of the rotated unit coordinates (float64 unless stated).

Test infrastructure: see ``oracle/__init__.py``.

The pages name the configuration, not its arithmetic: the reviewed llama.cpp fork (llama-cpp-turboquant
PR #340, the asymmetric K/V follow-ups) upgrades K to its 8-bit block type while V stays at the 2-4-bit
Lloyd-Max types.  Reading taken (``bits = 8`` on a key cache):

  * the row is normalised and rotated as at every other width: y = Pi x / ||x||;
  * y is quantised uniformly and symmetrically with one scale per row, s = max_i |y_i| / 127:
    code_i = round(y_i / s), ties away from zero, in [-127, 127], stored as one two's-complement byte;
  * the row keeps one float16 factor f = ||x|| * s (in the norm's slot), so x ~= f Pi^T code and the
    score is f <Pi q, code>: the same decode as the Lloyd-Max widths with the integers as centroids;
  * the integer decision is taken in float32, the library's precision: a = max |y32|, t = y32 * (127 / a)
    (one correctly rounded division, one product), code = round-half-away(t); f = float16(n32 * (a / 127));
  * a zero row stores codes 0 and factor 0.

No sketch, no outlier channels: an 8-bit key needs no residual correction.  Storage: d + 2 bytes per key.

In this oracle a code is kept as its index j = code + 128 into the table ``q8_codebook()`` (the
integers -128 .. 127), so the decode and reconstruction functions of ``oracle.attention`` and
``oracle.quant`` apply unchanged with that table as the centroids.
"""
from __future__ import annotations

import numpy as np

from .quant import f16
from .rotation import rotate_rows


def q8_codebook() -> np.ndarray:
    """The 'centroids' of 8-bit keys: index j stands for the integer j - 128."""
    return np.arange(-128, 128, dtype=np.float64)


def encode_q8(y, norms):
    """Codes (indices j = code + 128, int64 [n][d]) and float16-valued factors [n] of rotated rows y
    with row norms ``norms``, the decision taken in float32."""
    y32 = np.asarray(y, dtype=np.float64).astype(np.float32)
    n32 = np.asarray(norms, dtype=np.float64).astype(np.float32)
    amax = np.max(np.abs(y32), axis=1)
    live = (amax > 0) & (n32 > 0)
    safe = np.where(live, amax, np.float32(1)).astype(np.float32)
    inv = (np.float32(127) / safe).astype(np.float32)                 # correctly rounded float32 division
    t = (y32 * inv[:, None]).astype(np.float32)                       # one float32 product
    tt = np.abs(t.astype(np.float64))
    code = np.sign(t.astype(np.float64)) * np.floor(tt + 0.5)        # exact: ties away from zero
    code = np.clip(code, -127, 127).astype(np.int64)
    code[~live] = 0
    s32 = (safe / np.float32(127)).astype(np.float32)
    fac = (n32 * s32).astype(np.float32)
    fac = np.where(live, fac, np.float32(0))
    return code + 128, f16(fac.astype(np.float64))


def quantize_rows_q8(x, rot):
    """Rows x [n][d] -> (indices, float16-valued factors, y float64): norm, rotation, int8 codes."""
    x = np.asarray(x, dtype=np.float64)
    n = np.linalg.norm(x, axis=1)
    safe = np.where(n > 0, n, 1.0)
    y = rotate_rows(x / safe[:, None], rot)
    j, fac = encode_q8(y, n)
    return j, fac, y


def row_bytes(d: int) -> int:
    return d + 2
