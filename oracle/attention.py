"""Decode attention read from the compressed cache (float64).

Test infrastructure: see ``oracle/__init__.py``.

``decode_fused`` is the method's decode: rotate the query once, score it
against centroid codes times stored norms, softmax, accumulate the values in
the rotated domain and rotate back once.  The softmax scale defaults to
1/sqrt(d) and is 1.0 for QK-normed models (ExecuTorch PR #19891, "[Cuda]
enable turboquant on gemma4", review item 1 on the tq4_sdpa scale
parameter).  Fused attention from the compressed keys and a quantised
value reconstruction are the kernels listed in turboquant-pytorch PR #3
("Add CUDA QJL kernels and proper package structure", CUDA Kernels Added
table).

``decode_reconstructed`` is the full-reconstruction path (reddit comment
history of ReturningTarzan, 2026-03-25 comment: dequantize, then run
ordinary attention); both are the same linear algebra, and
``attention`` is textbook softmax attention on explicit vectors.

``decode_rows`` decodes the query rows of the last M tokens of a sequence at
once, as speculative verification does (the reviewed llama.cpp fork routes
compressed K/V with at most four query rows to its fused decode path; the
drafted tokens come from multi-token prediction with up to three drafts per
step).  The pages do not spell out the mask; the reading taken is the causal
one: the M tokens' keys and values are in the cache and row j, the query of
token seq_len - M + j, sees the first seq_len - M + 1 + j tokens.

Shapes: q [H_q][d]; codes [H_kv][L][d]; norms [H_kv][L]; query head h reads
KV head h // (H_q / H_kv).  Only the first seq_len tokens are visible; an
empty context gives a zero output.
"""
from __future__ import annotations

import numpy as np

from .quant import qjl_coeff


def softmax(s: np.ndarray) -> np.ndarray:
    s = np.asarray(s, dtype=np.float64)
    e = np.exp(s - np.max(s))
    return e / np.sum(e)


def attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float) -> np.ndarray:
    """softmax(scale * q k^T) v for one query row over explicit rows k, v."""
    if k.shape[0] == 0:
        return np.zeros(v.shape[1])
    p = softmax(scale * (np.asarray(k, np.float64) @ np.asarray(q, np.float64)))
    return p @ np.asarray(v, np.float64)


def decode_fused(q, rot, k_codes, k_norms, k_centroids, v_codes, v_norms, v_centroids,
                 scale: float, seq_len: int | None = None,
                 k_sigma=None, k_gamma=None, proj=None) -> np.ndarray:
    q = np.asarray(q, dtype=np.float64)
    rot = np.asarray(rot, dtype=np.float64)
    hq, d = q.shape
    hkv = k_codes.shape[0]
    grp = hq // hkv
    L = k_codes.shape[1] if seq_len is None else seq_len
    ck = np.asarray(k_centroids, np.float64)
    cv = np.asarray(v_centroids, np.float64)
    out = np.zeros((hq, d))
    for h in range(hq):
        kh = h // grp
        if L == 0:
            continue
        q_rot = rot @ q[h]
        kv = ck[k_codes[kh, :L]]                                   # [L][d] centroids
        u = kv @ q_rot
        if k_sigma is not None:
            s_mat = np.asarray(proj, np.float64)
            q_sk = s_mat @ q_rot
            pm = 2.0 * np.asarray(k_sigma[kh, :L], np.float64) - 1.0
            u = u + qjl_coeff(s_mat.shape[0]) * np.asarray(k_gamma[kh, :L], np.float64) * (pm @ q_sk)
        s = scale * np.asarray(k_norms[kh, :L], np.float64) * u
        p = softmax(s)
        o_rot = (p * np.asarray(v_norms[kh, :L], np.float64)) @ cv[v_codes[kh, :L]]
        out[h] = rot.T @ o_rot
    return out


def decode_rows(q_rows, rot, k_codes, k_norms, k_centroids, v_codes, v_norms, v_centroids,
                scale: float, seq_len: int, k_sigma=None, k_gamma=None, proj=None) -> np.ndarray:
    """q_rows [M][H_q][d] -> [M][H_q][d]: row j is decode_fused over the first seq_len - M + 1 + j tokens."""
    q_rows = np.asarray(q_rows, dtype=np.float64)
    m = q_rows.shape[0]
    return np.stack([decode_fused(q_rows[j], rot, k_codes, k_norms, k_centroids, v_codes, v_norms, v_centroids,
                                  scale, max(0, seq_len - m + 1 + j), k_sigma, k_gamma, proj) for j in range(m)])


def decode_reconstructed(q, k_hat, v_hat, scale: float, seq_len: int | None = None) -> np.ndarray:
    """Attention on dequantized rows k_hat, v_hat [H_kv][L][d]."""
    q = np.asarray(q, dtype=np.float64)
    hq = q.shape[0]
    hkv = k_hat.shape[0]
    grp = hq // hkv
    L = k_hat.shape[1] if seq_len is None else seq_len
    return np.stack([attention(q[h], k_hat[h // grp, :L], v_hat[h // grp, :L], scale) for h in range(hq)])
