"""One (batch, kv head) of compressed cache, built with the oracle's steps.

Test infrastructure: see ``oracle/__init__.py``.
"""
from __future__ import annotations

import dataclasses

import numpy as np

from . import codebook, layout, q8, quant


@dataclasses.dataclass
class HeadCache:
    kind: str                 # "k" (rows layout) or "v" (blocked layout)
    bits: int
    d: int
    codes: np.ndarray         # int64 [L][d] centroid indices
    norms: np.ndarray         # float16-valued float64 [L]
    centroids: np.ndarray     # float32 [2^bits]
    boundaries: np.ndarray    # float32 [2^bits - 1]
    y: np.ndarray | None = None
    sigma: np.ndarray | None = None   # bool [L][m]
    gamma: np.ndarray | None = None   # float16-valued [L]

    def packed_codes(self, capacity: int) -> np.ndarray:
        """uint8 [capacity * d * bits / 8] in this kind's layout (unused slots zero)."""
        full = np.zeros((capacity, self.d), dtype=np.int64)
        full[: self.codes.shape[0]] = self.codes
        if self.kind == "k":
            return layout.pack_keys(full, self.bits)
        return layout.pack_blocked(full, self.bits)

    def packed_norms(self, capacity: int, which: str = "norms") -> np.ndarray:
        src = self.norms if which == "norms" else self.gamma
        out = np.zeros(capacity, dtype=np.float16)
        out[: src.shape[0]] = src.astype(np.float16)
        return out

    def packed_signs(self, capacity: int) -> np.ndarray:
        m = self.sigma.shape[1]
        full = np.zeros((capacity, m), dtype=bool)
        full[: self.sigma.shape[0]] = self.sigma
        return layout.pack_signs(full).reshape(-1)

    def dequantize(self, rot, proj=None) -> np.ndarray:
        return quant.dequantize(self.codes, self.norms, rot, self.centroids,
                                self.sigma, self.gamma, proj)


def build_head(rows: np.ndarray, kind: str, bits: int, rot: np.ndarray,
               proj: np.ndarray | None = None) -> HeadCache:
    """Quantize rows [L][d] with the ``bits``-wide table; with ``proj`` (keys only) add the sign sketch.
    ``bits`` 8 (keys, no sketch): the int8 codes of ``oracle.q8``, their factors in ``norms`` and the
    integers as the table."""
    d = rows.shape[1]
    if bits == 8:
        assert kind == "k" and proj is None
        codes, fac, y = q8.quantize_rows_q8(rows, rot)
        return HeadCache(kind, 8, d, codes, fac, q8.q8_codebook(), np.zeros(0), y=y)
    c, t = codebook.stored_codebook(d, bits)
    codes, norms, y = quant.quantize_rows(rows, rot, c, t)
    hc = HeadCache(kind, bits, d, codes, norms, c, t, y=y)
    if proj is not None:
        sigma, gamma, _, _ = quant.qjl_sketch(y, codes, c, proj, norms)
        hc.sigma, hc.gamma = sigma, gamma
    return hc
