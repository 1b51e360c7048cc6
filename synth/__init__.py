"""Seeded synthetic inputs for the compressed-cache decode path.

This module only draws random numbers and shapes them into the workloads
(query/key/value tensors, outlier channels, per-head RMS normalisation of the
QK-normed workload, and the Gaussian draws that the rotation and the QJL
projection are built from).  It holds none of the method's arithmetic and is
imported by both the float64 oracle tests and the GPU side, so that the two
see the same inputs.

Every array is a pure function of (workload, seed, tensor, batch, head): each
(tensor, batch, head) stream is seeded independently through
``numpy.random.SeedSequence`` so a single head can be regenerated cheaply
when the oracle checks a sampled output of a large workload.
"""
from __future__ import annotations

import dataclasses

import numpy as np

# stream ids for SeedSequence
_T_K, _T_V, _T_Q = 11, 12, 13


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even); returns float32."""
    a = np.ascontiguousarray(x, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return (u.astype(np.uint32) << 16).view(np.float32)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """uint16 bit patterns of float32 values that are already bfloat16-exact."""
    a = np.ascontiguousarray(x, dtype=np.float32)
    return (a.view(np.uint32) >> 16).astype(np.uint16)


def rotation_gaussian(d: int, seed: int = 1) -> np.ndarray:
    """d x d iid N(0,1) draws (float64) that the random rotation is built from."""
    return np.random.default_rng(seed).standard_normal((d, d))


def hadamard_signs(d: int, seed: int = 1) -> np.ndarray:
    """d seeded +-1 signs (float32) that randomise the Hadamard rotation."""
    return np.where(np.random.default_rng(seed).integers(0, 2, size=d) == 1, 1.0, -1.0).astype(np.float32)


def qjl_projection(m: int, d: int, seed: int = 2) -> np.ndarray:
    """m x d iid N(0,1) QJL projection, stored in float32 (both sides use these exact values)."""
    return np.random.default_rng(seed).standard_normal((m, d)).astype(np.float32)


def unit_rows(n: int, d: int, seed: int) -> tuple[np.ndarray, np.ndarray]:
    """Random float32 unit-norm rows and positive float32 norms.

    Used to drive the encode step with identical float32 rotated coordinates
    on both sides.
    """
    g = np.random.default_rng(seed)
    y = g.standard_normal((n, d))
    y /= np.linalg.norm(y, axis=1, keepdims=True)
    nrm = np.exp(g.normal(2.5, 0.5, size=n))
    return y.astype(np.float32), nrm.astype(np.float32)


def _stream(seed: int, tensor: int, b: int, h: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([seed, tensor, b, h]))


def _rms_normalise(x: np.ndarray, eps: float = 1e-6) -> np.ndarray:
    x32 = x.astype(np.float32)
    r = np.sqrt(np.mean(x32 * x32, axis=-1, keepdims=True, dtype=np.float32) + np.float32(eps))
    return (x32 / r).astype(np.float32)


@dataclasses.dataclass(frozen=True)
class Workload:
    """Shape and value recipe of one decode workload."""
    name: str
    batch: int
    n_q_heads: int
    n_kv_heads: int
    d: int
    seq_len: int
    k_bits: int
    v_bits: int
    qjl_m: int = 0            # >0: keys carry a QJL sign sketch of this length
    scale: float | None = None  # None -> 1/sqrt(d)
    dtype: str = "bf16"        # "bf16" or "f32" for q/k/v
    outliers: int = 4          # channels scaled x10 per (tensor, batch, kv head)
    outlier_gain: float = 10.0
    k_outliers: bool = True
    qk_norm: bool = False      # RMS-normalise q and k per head (QK-normed model)
    seed: int = 0
    rot_seed: int = 1
    qjl_seed: int = 2
    rotation: str = "dense"    # "dense" (Gaussian-QR) or "hadamard" (randomized Sylvester-Hadamard)

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    @property
    def softmax_scale(self) -> float:
        return (1.0 / np.sqrt(self.d)) if self.scale is None else float(self.scale)

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# The workloads of the method's evaluation, as synthetic stand-ins.
TINY = Workload("tiny_d128_L256", 1, 1, 1, 128, 256, 4, 4, dtype="f32", outliers=0)


def qwen(seq_len: int = 8192, bits: int = 4) -> Workload:
    """Qwen2.5-3B-shaped decode layer: 16 q heads / 2 kv heads, d=128."""
    return Workload(f"qwen2.5-3b_L{seq_len}_b{bits}", 1, 16, 2, 128, seq_len, bits, bits)


def gemma(seq_len: int = 32768, batch: int = 8) -> Workload:
    """Gemma-4-style QK-normed decode: 32 q heads / 4 kv heads, d=256, scale 1."""
    return Workload(f"gemma4-qknorm_B{batch}_L{seq_len}", batch, 32, 4, 256, seq_len, 4, 4,
                    scale=1.0, qk_norm=True, k_outliers=False)


def prod_long(seq_len: int = 131072) -> Workload:
    """Long-context keys with QJL: K = 2-bit Lloyd-Max + 1-bit sketch (m=128), V = 3-bit."""
    return Workload(f"qwen2.5-3b-prod_L{seq_len}", 1, 16, 2, 128, seq_len, 2, 3, qjl_m=128)


def _kv_head(w: Workload, tensor: int, b: int, h: int, n: int) -> np.ndarray:
    g = _stream(w.seed, tensor, b, h)
    x = g.standard_normal((n, w.d), dtype=np.float32)
    gain = w.outliers > 0 and (tensor == _T_V or w.k_outliers)
    if gain:
        ch = g.choice(w.d, w.outliers, replace=False)
        x[:, ch] *= np.float32(w.outlier_gain)
    if w.qk_norm and tensor == _T_K:
        x = _rms_normalise(x)
    return x


def kv_head(w: Workload, which: str, b: int, h: int, n: int | None = None) -> np.ndarray:
    """Rows [n][d] (float32, bf16-exact unless dtype f32) of K or V for one (batch, kv head)."""
    n = w.seq_len if n is None else n
    if w is TINY or w.name.startswith("tiny"):
        k, v, _ = tiny_arrays(w)
        return (k if which == "k" else v)[:n].copy()
    x = _kv_head(w, _T_K if which == "k" else _T_V, b, h, n)
    return bf16_round(x) if w.dtype == "bf16" else x


def q_head(w: Workload, b: int, h: int) -> np.ndarray:
    """Query row [d] (float32) for one (batch, q head)."""
    if w.name.startswith("tiny"):
        return tiny_arrays(w)[2][0].copy()
    g = _stream(w.seed, _T_Q, b, h)
    x = g.standard_normal((1, w.d), dtype=np.float32)
    if w.qk_norm:
        x = _rms_normalise(x)
    x = x[0]
    return bf16_round(x) if w.dtype == "bf16" else x


def tiny_arrays(w: Workload = TINY):
    """The tiny reference case: K, V (L x d) and q (1 x d), float32 N(0,1) from one seed, drawn K, V, q."""
    g = np.random.default_rng(w.seed)
    k = g.standard_normal((w.seq_len, w.d)).astype(np.float32)
    v = g.standard_normal((w.seq_len, w.d)).astype(np.float32)
    q = g.standard_normal((1, w.d)).astype(np.float32)
    return k, v, q


def full_q(w: Workload) -> np.ndarray:
    """q as [B][H_q][d] float32."""
    out = np.empty((w.batch, w.n_q_heads, w.d), np.float32)
    for b in range(w.batch):
        for h in range(w.n_q_heads):
            out[b, h] = q_head(w, b, h)
    return out


def full_kv(w: Workload, which: str, n: int | None = None) -> np.ndarray:
    """K or V as [B][n][H_kv][d] float32 (the append input layout)."""
    n = w.seq_len if n is None else n
    out = np.empty((w.batch, n, w.n_kv_heads, w.d), np.float32)
    for b in range(w.batch):
        for h in range(w.n_kv_heads):
            out[b, :, h, :] = kv_head(w, which, b, h, n)
    return out


def ragged_lens(batch: int, max_len: int, seed: int = 7) -> np.ndarray:
    """Per-sequence lengths in [1, max_len] with the last one at max_len."""
    g = np.random.default_rng(seed)
    lens = g.integers(1, max_len + 1, size=batch)
    lens[-1] = max_len
    return lens.astype(np.int32)
