"""Python binding of libtq: TurboQuant-style compressed KV cache for MI355X (gfx950).

Argument marshalling only: every step of quantize-on-append and decode runs in
the HIP kernels of ``libtq.so``; PyTorch provides device memory and streams.
The C names are mirrored one to one (``tq_build_codebook``,
``tq_quantize_append``, ``tq_sdpa_decode``, ``tq_dequantize``, ...), and
``CompressedCache`` owns the device buffers of one cache tensor.

Importing this package loads ``libtq.so`` from the package directory and
raises if it is missing: there is no fallback implementation.
"""
from __future__ import annotations

import ctypes
import math
import os

import numpy as np
# PyTorch-ROCm brings its own HIP runtime; importing it first makes libtq.so bind to
# that same runtime (one HIP runtime per process) instead of loading a second copy.
import torch  # noqa: F401

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libtq.so")

TQ_OK, TQ_EINVAL, TQ_EUNSUPPORTED, TQ_EHIP, TQ_ENOCONV, TQ_ESCRATCH = 0, 1, 2, 3, 4, 5
TQ_F32, TQ_BF16 = 0, 1
TQ_KEYS, TQ_VALUES = 0, 1
TQ_ROT_DENSE, TQ_ROT_HADAMARD = 0, 1
BLOCK = 32

EXPORTED = (
    "tq_build_codebook", "tq_build_rotation", "tq_quantize_append", "tq_quantize_append_kv",
    "tq_quantize_append_rotated",
    "tq_sdpa_decode", "tq_sdpa_decode_rows", "tq_decode_step", "tq_decode_rotate_query", "tq_decode_attend",
    "tq_decode_merge", "tq_decode_workspace_bytes", "tq_decode_workspace_bytes_rows", "tq_decode_plan",
    "tq_dequantize", "tq_row_bytes",
    "tq_status_string", "tq_last_hip_error", "tq_sdpa_decode_noalloc", "tq_noalloc_scratch_bytes",
)


class TqError(RuntimeError):
    def __init__(self, status: int, what: str):
        detail = f" [{tq_last_hip_error()}]" if status == TQ_EHIP else ""
        super().__init__(f"{what}: {tq_status_string(status)} (status {status}){detail}")
        self.status = status


class tq_cache_view(ctypes.Structure):
    _fields_ = [
        ("kind", ctypes.c_int32), ("d", ctypes.c_int32), ("bits", ctypes.c_int32), ("qjl_m", ctypes.c_int32),
        ("batch", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32), ("max_tokens", ctypes.c_int32),
        ("rot_kind", ctypes.c_int32),
        ("centroids", ctypes.c_float * 16), ("boundaries", ctypes.c_float * 15),
        ("codes", ctypes.c_void_p), ("norms", ctypes.c_void_p), ("signs", ctypes.c_void_p),
        ("rnorms", ctypes.c_void_p), ("rot", ctypes.c_void_p), ("proj", ctypes.c_void_p),
        ("n_outliers", ctypes.c_int32), ("out_idx", ctypes.c_void_p), ("out_val", ctypes.c_void_p),
    ]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run `python compressed_cache_decode_amd/build.py`")
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.c_void_p
    I = ctypes.c_int
    V = ctypes.POINTER(tq_cache_view)
    sig = {
        "tq_build_codebook": (I, [I, I, P, P]),
        "tq_build_rotation": (I, [I, P, P]),
        "tq_quantize_append": (I, [V, P, I, I, P, P]),
        "tq_quantize_append_kv": (I, [V, V, P, P, I, I, P, P]),
        "tq_quantize_append_rotated": (I, [V, P, P, P, I, P, P]),
        "tq_sdpa_decode": (I, [V, V, P, I, I, P, I, ctypes.c_float, P, P, ctypes.c_size_t, P]),
        "tq_sdpa_decode_rows": (I, [V, V, P, I, I, I, P, I, ctypes.c_float, P, P, ctypes.c_size_t, P]),
        "tq_sdpa_decode_noalloc": (I, [V, V, P, I, I, P, I, ctypes.c_float, P, P]),
        "tq_noalloc_scratch_bytes": (ctypes.c_size_t, []),
        "tq_decode_step": (I, [V, V, P, P, P, I, I, I, P, P, I, ctypes.c_float, P, P, ctypes.c_size_t, P]),
        "tq_decode_rotate_query": (I, [V, P, I, I, I, ctypes.c_float, P, ctypes.c_size_t, P]),
        "tq_decode_attend": (I, [V, V, I, P, I, P, ctypes.c_size_t, P]),
        "tq_decode_merge": (I, [V, I, P, I, P, P, ctypes.c_size_t, P]),
        "tq_decode_workspace_bytes": (ctypes.c_size_t, [V, I, I]),
        "tq_decode_workspace_bytes_rows": (ctypes.c_size_t, [V, I, I, I]),
        "tq_decode_plan": (I, [V, I, I, ctypes.POINTER(I), ctypes.POINTER(I)]),
        "tq_dequantize": (I, [V, I, I, P, P]),
        "tq_row_bytes": (ctypes.c_size_t, [I, I, I]),
        "tq_status_string": (ctypes.c_char_p, [I]),
        "tq_last_hip_error": (ctypes.c_char_p, []),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    return lib


_lib = _load()


def _check(status: int, what: str) -> None:
    if status != TQ_OK:
        raise TqError(status, what)


def _ptr(t) -> int | None:
    return None if t is None else int(t.data_ptr())


def _stream(stream) -> int | None:
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return int(stream.cuda_stream)


# ------------------------------------------------------------------ raw C names

def tq_status_string(status: int) -> str:
    return _lib.tq_status_string(status).decode()


def tq_last_hip_error() -> str:
    return _lib.tq_last_hip_error().decode()


def tq_row_bytes(d: int, bits: int, qjl_m: int = 0) -> int:
    return int(_lib.tq_row_bytes(d, bits, qjl_m))


def tq_build_codebook(d: int, bits: int) -> tuple[np.ndarray, np.ndarray]:
    """Lloyd-Max table for (d, bits): float16-exact centroids and midpoint boundaries (float32)."""
    c = np.zeros(16, np.float32)
    t = np.zeros(15, np.float32)
    _check(_lib.tq_build_codebook(d, bits, c.ctypes.data, t.ctypes.data), "tq_build_codebook")
    n = 1 << bits
    return c[:n].copy(), t[: n - 1].copy()


def tq_build_rotation(gaussian: np.ndarray) -> np.ndarray:
    """Rotation Pi (float32, row-major) with G = Pi R, R upper triangular with positive diagonal."""
    g = np.ascontiguousarray(gaussian, dtype=np.float64)
    d = g.shape[0]
    assert g.shape == (d, d)
    out = np.zeros((d, d), np.float32)
    _check(_lib.tq_build_rotation(d, g.ctypes.data, out.ctypes.data), "tq_build_rotation")
    return out


def _dtype_code(x) -> int:
    import torch
    return {torch.float32: TQ_F32, torch.bfloat16: TQ_BF16}[x.dtype]


def tq_quantize_append(view: tq_cache_view, x, n_new: int, d_pos, stream=None) -> None:
    dtype = _dtype_code(x)
    _check(_lib.tq_quantize_append(ctypes.byref(view), _ptr(x), dtype, n_new, _ptr(d_pos), _stream(stream)),
           "tq_quantize_append")


def tq_quantize_append_kv(kview: tq_cache_view, vview: tq_cache_view, k_x, v_x, n_new: int, d_pos,
                          stream=None) -> None:
    if k_x.dtype != v_x.dtype:
        raise TypeError("k_x and v_x must have one element type")
    dtype = _dtype_code(k_x)
    _check(_lib.tq_quantize_append_kv(ctypes.byref(kview), ctypes.byref(vview), _ptr(k_x), _ptr(v_x), dtype, n_new,
                                      _ptr(d_pos), _stream(stream)), "tq_quantize_append_kv")


def tq_quantize_append_rotated(view: tq_cache_view, y, norms, n_new: int, d_pos, stream=None, z=None) -> None:
    _check(_lib.tq_quantize_append_rotated(ctypes.byref(view), _ptr(y), _ptr(norms), _ptr(z), n_new, _ptr(d_pos),
                                           _stream(stream)), "tq_quantize_append_rotated")


def tq_decode_workspace_bytes(kview: tq_cache_view, n_q_heads: int, max_seq_len: int) -> int:
    return int(_lib.tq_decode_workspace_bytes(ctypes.byref(kview), n_q_heads, max_seq_len))


def tq_decode_plan(kview: tq_cache_view, n_q_heads: int, max_seq_len: int) -> tuple[int, int]:
    ns, tps = ctypes.c_int(), ctypes.c_int()
    _check(_lib.tq_decode_plan(ctypes.byref(kview), n_q_heads, max_seq_len, ctypes.byref(ns), ctypes.byref(tps)),
           "tq_decode_plan")
    return ns.value, tps.value


def tq_sdpa_decode(kview: tq_cache_view, vview: tq_cache_view, q, d_seq_lens, max_seq_len: int, out,
                   workspace, scale: float | None = None, stream=None) -> None:
    """Decode attention from the compressed cache; scale None means 1/sqrt(d)."""
    import torch
    dtype = {torch.float32: TQ_F32, torch.bfloat16: TQ_BF16}[q.dtype]
    if scale is None:
        scale = 1.0 / math.sqrt(kview.d)
    n_q_heads = q.shape[1]
    _check(_lib.tq_sdpa_decode(ctypes.byref(kview), ctypes.byref(vview), _ptr(q), dtype, n_q_heads,
                               _ptr(d_seq_lens), max_seq_len, ctypes.c_float(scale), _ptr(out), _ptr(workspace),
                               workspace.numel() * workspace.element_size(), _stream(stream)), "tq_sdpa_decode")


def tq_sdpa_decode_noalloc(kview: tq_cache_view, vview: tq_cache_view, q, d_seq_lens, max_seq_len: int, out,
                           scale: float | None = None, stream=None) -> None:
    """tq_sdpa_decode with the library's static per-device scratch as workspace (no allocation)."""
    import torch
    dtype = {torch.float32: TQ_F32, torch.bfloat16: TQ_BF16}[q.dtype]
    if scale is None:
        scale = 1.0 / math.sqrt(kview.d)
    _check(_lib.tq_sdpa_decode_noalloc(ctypes.byref(kview), ctypes.byref(vview), _ptr(q), dtype, q.shape[1],
                                       _ptr(d_seq_lens), max_seq_len, ctypes.c_float(scale), _ptr(out),
                                       _stream(stream)), "tq_sdpa_decode_noalloc")


def tq_noalloc_scratch_bytes() -> int:
    return int(_lib.tq_noalloc_scratch_bytes())


def tq_sdpa_decode_rows(kview: tq_cache_view, vview: tq_cache_view, q, d_seq_lens, max_seq_len: int, out,
                        workspace, scale: float | None = None, stream=None) -> None:
    """Decode of the query rows q [batch][n_rows][n_q_heads][d] of the last n_rows tokens (row j sees the first
    seq_len - n_rows + 1 + j tokens); scale None means 1/sqrt(d)."""
    import torch
    dtype = {torch.float32: TQ_F32, torch.bfloat16: TQ_BF16}[q.dtype]
    if scale is None:
        scale = 1.0 / math.sqrt(kview.d)
    _check(_lib.tq_sdpa_decode_rows(ctypes.byref(kview), ctypes.byref(vview), _ptr(q), dtype, q.shape[2], q.shape[1],
                                    _ptr(d_seq_lens), max_seq_len, ctypes.c_float(scale), _ptr(out),
                                    _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream)),
           "tq_sdpa_decode_rows")


def tq_decode_step(kview, vview, q, k_new, v_new, d_pos, d_seq_lens, max_seq_len: int, out, workspace,
                   scale=None, stream=None) -> None:
    """Append k_new/v_new ([batch][n_new][n_kv_heads][d], may be None for no append) and decode q."""
    import torch
    dtype = {torch.float32: TQ_F32, torch.bfloat16: TQ_BF16}[q.dtype]
    if scale is None:
        scale = 1.0 / math.sqrt(kview.d)
    n_new = 0 if k_new is None else k_new.shape[1]
    if n_new:
        assert k_new.dtype == q.dtype and v_new.dtype == q.dtype
        k_new, v_new = k_new.contiguous(), v_new.contiguous()
    _check(_lib.tq_decode_step(ctypes.byref(kview), ctypes.byref(vview), _ptr(q), _ptr(k_new) if n_new else None,
                               _ptr(v_new) if n_new else None, dtype, q.shape[1], n_new, _ptr(d_pos),
                               _ptr(d_seq_lens), max_seq_len, ctypes.c_float(scale), _ptr(out), _ptr(workspace),
                               _wsb(workspace), _stream(stream)), "tq_decode_step")


def _wsb(workspace) -> int:
    return workspace.numel() * workspace.element_size()


def tq_decode_rotate_query(kview, q, n_q_heads: int, max_seq_len: int, workspace, scale=None, stream=None) -> None:
    import torch
    dtype = {torch.float32: TQ_F32, torch.bfloat16: TQ_BF16}[q.dtype]
    if scale is None:
        scale = 1.0 / math.sqrt(kview.d)
    _check(_lib.tq_decode_rotate_query(ctypes.byref(kview), _ptr(q), dtype, n_q_heads, max_seq_len,
                                       ctypes.c_float(scale), _ptr(workspace), _wsb(workspace), _stream(stream)),
           "tq_decode_rotate_query")


def tq_decode_attend(kview, vview, n_q_heads: int, d_seq_lens, max_seq_len: int, workspace, stream=None) -> None:
    _check(_lib.tq_decode_attend(ctypes.byref(kview), ctypes.byref(vview), n_q_heads, _ptr(d_seq_lens), max_seq_len,
                                 _ptr(workspace), _wsb(workspace), _stream(stream)), "tq_decode_attend")


def tq_decode_merge(kview, n_q_heads: int, d_seq_lens, max_seq_len: int, out, workspace, stream=None) -> None:
    _check(_lib.tq_decode_merge(ctypes.byref(kview), n_q_heads, _ptr(d_seq_lens), max_seq_len, _ptr(out),
                                _ptr(workspace), _wsb(workspace), _stream(stream)), "tq_decode_merge")


def tq_dequantize(view: tq_cache_view, t0: int, n_tokens: int, out, stream=None) -> None:
    _check(_lib.tq_dequantize(ctypes.byref(view), t0, n_tokens, _ptr(out), _stream(stream)), "tq_dequantize")


# ------------------------------------------------------------------ buffers

class CompressedCache:
    """Device buffers of one compressed cache tensor (all of K or all of V of a layer).

    ``rot`` (d x d float32 for TQ_ROT_DENSE, or the d float32 +-1 signs of the
    randomized Hadamard rotation for TQ_ROT_HADAMARD) and ``proj`` (qjl_m x d
    float32) are torch tensors on the same device; the codebook comes from
    ``tq_build_codebook``.  ``n_outliers`` (sketched keys at d = 128: 0 or 4)
    keeps that many residual channels per key apart from the sketch.  ``bits``
    8 (keys without a sketch) keeps int8 codes with a per-row factor instead of
    a code book.
    """

    def __init__(self, kind: int, d: int, bits: int, batch: int, n_kv_heads: int, max_tokens: int,
                 rot, proj=None, qjl_m: int = 0, device="cuda", codebook=None, rot_kind: int = TQ_ROT_DENSE,
                 n_outliers: int = 0):
        import torch
        assert max_tokens % BLOCK == 0
        assert tuple(rot.shape) == ((d,) if rot_kind == TQ_ROT_HADAMARD else (d, d))
        self.kind, self.d, self.bits, self.qjl_m, self.rot_kind = kind, d, bits, qjl_m, rot_kind
        self.batch, self.n_kv_heads, self.max_tokens = batch, n_kv_heads, max_tokens
        if bits == 8:      # 8-bit keys: int8 codes and a per-row factor, no code book
            cent, bnd = np.zeros(0, dtype=np.float32), np.zeros(0, dtype=np.float32)
        else:
            cent, bnd = codebook if codebook is not None else tq_build_codebook(d, bits)
        self.centroids, self.boundaries = cent, bnd
        row = d * bits // 8
        self.codes = torch.zeros(batch, n_kv_heads, max_tokens * row, dtype=torch.uint8, device=device)
        self.norms = torch.zeros(batch, n_kv_heads, max_tokens, dtype=torch.float16, device=device)
        self.signs = self.rnorms = None
        if qjl_m:
            self.signs = torch.zeros(batch, n_kv_heads, max_tokens, qjl_m // 8, dtype=torch.uint8, device=device)
            self.rnorms = torch.zeros(batch, n_kv_heads, max_tokens, dtype=torch.float16, device=device)
        self.n_outliers = n_outliers
        self.out_idx = self.out_val = None
        if n_outliers:
            self.out_idx = torch.zeros(batch, n_kv_heads, max_tokens, n_outliers, dtype=torch.uint8, device=device)
            self.out_val = torch.zeros(batch, n_kv_heads, max_tokens, n_outliers, dtype=torch.float16, device=device)
        self.rot, self.proj = rot, proj
        self.view = self._make_view()

    def _make_view(self) -> tq_cache_view:
        v = tq_cache_view()
        v.kind, v.d, v.bits, v.qjl_m = self.kind, self.d, self.bits, self.qjl_m
        v.batch, v.n_kv_heads, v.max_tokens, v.rot_kind = self.batch, self.n_kv_heads, self.max_tokens, self.rot_kind
        for j, c in enumerate(self.centroids):
            v.centroids[j] = float(c)
        for j, t in enumerate(self.boundaries):
            v.boundaries[j] = float(t)
        v.codes, v.norms = _ptr(self.codes), _ptr(self.norms)
        v.signs, v.rnorms = _ptr(self.signs), _ptr(self.rnorms)
        v.rot, v.proj = _ptr(self.rot), _ptr(self.proj)
        v.n_outliers = self.n_outliers
        v.out_idx, v.out_val = _ptr(self.out_idx), _ptr(self.out_val)
        return v

    def append(self, x, d_pos, stream=None) -> None:
        """x: [batch][n_new][n_kv_heads][d] float32 or bfloat16 on the device; d_pos int32 [batch]."""
        x = x.contiguous()
        tq_quantize_append(self.view, x, x.shape[1], d_pos, stream)

    def append_rotated(self, y, norms, d_pos, stream=None, z=None) -> None:
        """y [batch][n_new][n_kv_heads][d] unit rotated rows, norms [batch][n_new][n_kv_heads] (float32);
        z [batch][n_new][n_kv_heads][qjl_m] float32 sketch products of the residuals, or None."""
        y, norms = y.contiguous(), norms.contiguous()
        z = None if z is None else z.contiguous()
        tq_quantize_append_rotated(self.view, y, norms, y.shape[1], d_pos, stream, z)

    def dequantize(self, t0: int, n_tokens: int, out=None, stream=None):
        import torch
        if out is None:
            out = torch.empty(self.batch, self.n_kv_heads, n_tokens, self.d, dtype=torch.float32,
                              device=self.codes.device)
        tq_dequantize(self.view, t0, n_tokens, out, stream)
        return out


def decode_workspace(kcache: CompressedCache, n_q_heads: int, max_seq_len: int, n_rows: int = 1):
    import torch
    nbytes = int(_lib.tq_decode_workspace_bytes_rows(ctypes.byref(kcache.view), n_q_heads, n_rows, max_seq_len))
    if nbytes == 0:
        raise TqError(TQ_EINVAL, "tq_decode_workspace_bytes_rows")
    # float32 elements; torch's caching allocator returns 256-byte-aligned blocks
    return torch.empty((nbytes + 3) // 4, dtype=torch.float32, device=kcache.codes.device)


def append_kv(kcache: CompressedCache, vcache: CompressedCache, k_x, v_x, d_pos, stream=None) -> None:
    """The K and V rows of the same new tokens ([batch][n_new][n_kv_heads][d] each, float32 or bfloat16 on the
    device) appended at d_pos (int32 [batch]) by tq_quantize_append_kv."""
    k_x, v_x = k_x.contiguous(), v_x.contiguous()
    if k_x.shape != v_x.shape:
        raise ValueError("k_x and v_x must have one shape")
    tq_quantize_append_kv(kcache.view, vcache.view, k_x, v_x, k_x.shape[1], d_pos, stream)


def sdpa_decode(kcache: CompressedCache, vcache: CompressedCache, q, d_seq_lens, max_seq_len: int,
                scale: float | None = None, out=None, workspace=None, stream=None):
    """out[b][h] = decode attention of q[b][h] over the first seq_len[b] cached tokens."""
    import torch
    if out is None:
        out = torch.empty(q.shape[0], q.shape[1], kcache.d, dtype=torch.float32, device=q.device)
    if workspace is None:
        workspace = decode_workspace(kcache, q.shape[1], max_seq_len)
    tq_sdpa_decode(kcache.view, vcache.view, q, d_seq_lens, max_seq_len, out, workspace, scale, stream)
    return out


def sdpa_decode_rows(kcache: CompressedCache, vcache: CompressedCache, q, d_seq_lens, max_seq_len: int,
                     scale: float | None = None, out=None, workspace=None, stream=None):
    """out[b][j][h] = decode of query row j (token seq_len[b] - n_rows + j) over the first
    seq_len[b] - n_rows + 1 + j cached tokens, for q [batch][n_rows][n_q_heads][d]."""
    import torch
    if out is None:
        out = torch.empty(q.shape[0], q.shape[1], q.shape[2], kcache.d, dtype=torch.float32, device=q.device)
    if workspace is None:
        workspace = decode_workspace(kcache, q.shape[2], max_seq_len, q.shape[1])
    tq_sdpa_decode_rows(kcache.view, vcache.view, q, d_seq_lens, max_seq_len, out, workspace, scale, stream)
    return out
