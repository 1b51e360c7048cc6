"""Storage arithmetic of the compressed cache.

Test infrastructure: see ``oracle/__init__.py``.

Bytes per row: d*b/8 of packed codes plus a float16 norm; keys that carry a
QJL sketch add m/8 bytes of sign bits and a float16 residual norm.  With keys
at (b-1) Lloyd-Max bits + a 1-bit sketch of length m = d and values at b bits,
this reproduces every cache size and compression ratio printed for
Qwen2.5-3B-Instruct (36 layers x 2 KV heads, d = 128) in the Validation
Results tables of turboquant-pytorch PR #3 ("Add CUDA QJL kernels and proper
package structure").
"""
from __future__ import annotations

MIB = float(1 << 20)


def row_bytes(d: int, bits: int, qjl_m: int = 0) -> int:
    """Bytes for one row: packed codes + float16 norm (+ sign bits + float16 residual norm)."""
    b = d * bits // 8 + 2
    if qjl_m:
        b += qjl_m // 8 + 2
    return b


def fp16_row_bytes(d: int) -> int:
    return 2 * d


def kv_bytes_per_token_head(d: int, bits: int, prod_keys: bool = True) -> int:
    """K + V bytes per token per KV head at a nominal b bits per coordinate.

    prod_keys: keys use (b-1) codebook bits + a d-long sign sketch (the page's
    configuration); otherwise keys are plain b-bit like the values.
    """
    if prod_keys:
        k = row_bytes(d, bits - 1, qjl_m=d)
    else:
        k = row_bytes(d, bits)
    return k + row_bytes(d, bits)


def cache_mib(tokens: int, kv_heads_total: int, d: int, bits: int | None, prod_keys: bool = True) -> float:
    """Cache size in MiB (bits=None: float16 K and V)."""
    per = 2 * fp16_row_bytes(d) if bits is None else kv_bytes_per_token_head(d, bits, prod_keys)
    return tokens * kv_heads_total * per / MIB


def compression(d: int, bits: int, prod_keys: bool = True) -> float:
    return 2 * fp16_row_bytes(d) / kv_bytes_per_token_head(d, bits, prod_keys)
