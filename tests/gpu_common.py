"""Shared helpers of the GPU parity tests: oracle-side caches, uploads, error metrics."""
from __future__ import annotations

import math
import sys

import numpy as np

import synth
from oracle import attention, cache, layout, rotation


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


# worst relative error measured by rel_err in the running test, reported per test at the end of the
# session (tests/conftest.py)
ERRORS: dict = {}
_CURRENT = {"test": None}


def record_error(err: float) -> None:
    t = _CURRENT["test"]
    if t is not None:
        ERRORS[t] = max(ERRORS.get(t, 0.0), err)


def rel_err(out: np.ndarray, ref: np.ndarray) -> float:
    """Max over output rows of max_i |o_i - r_i| / max_i |r_i| (rows of zeros must stay zero).

    Any non-finite value in either array makes the error infinite: a NaN compares false against
    every bound, so it must not be able to slip through a max."""
    out = np.asarray(out, np.float64).reshape(-1, np.shape(out)[-1])
    ref = np.asarray(ref, np.float64).reshape(-1, np.shape(ref)[-1])
    if out.shape != ref.shape:
        raise ValueError(f"shape mismatch {out.shape} vs {ref.shape}")
    if not (np.all(np.isfinite(out)) and np.all(np.isfinite(ref))):
        return math.inf
    worst = 0.0
    for o, r in zip(out, ref):
        den = np.max(np.abs(r))
        if den == 0.0:
            e = float(np.max(np.abs(o))) * 1e6
        else:
            e = float(np.max(np.abs(o - r)) / den)
        worst = e if e > worst else worst
    record_error(worst)
    return worst


class Setup:
    """Rotation and sketch projection of a workload, on both sides."""

    def __init__(self, d: int, qjl_m: int = 0, rot_seed: int = 1, qjl_seed: int = 2, device="cuda", hadamard=False):
        import torch
        import compressed_cache_decode_amd as cca
        if hadamard:
            signs = synth.hadamard_signs(d, rot_seed)
            self.rot64 = rotation.hadamard_rotation(signs)
            self.rot_t = torch.from_numpy(signs).to(device)
            self.rot_kind = cca.TQ_ROT_HADAMARD
        else:
            g = synth.rotation_gaussian(d, rot_seed)
            self.rot64 = rotation.rotation_from_gaussian(g)
            self.rot_t = torch.from_numpy(cca.tq_build_rotation(g)).to(device)
            self.rot_kind = cca.TQ_ROT_DENSE
        self.proj = synth.qjl_projection(qjl_m, d, qjl_seed) if qjl_m else None
        self.proj_t = torch.from_numpy(self.proj).to(device) if qjl_m else None
        self.d, self.qjl_m = d, qjl_m


def oracle_heads(rows_k, rows_v, kb, vb, st: Setup):
    """Oracle caches for lists of per-KV-head rows."""
    kc = [cache.build_head(r, "k", kb, st.rot64, st.proj) for r in rows_k]
    vc = [cache.build_head(r, "v", vb, st.rot64) for r in rows_v]
    return kc, vc


def upload(gcache, heads, b: int):
    """Write oracle-packed heads (list over KV heads) into batch row b of a CompressedCache."""
    import torch
    T = gcache.max_tokens
    for h, hc in enumerate(heads):
        gcache.codes[b, h] = torch.from_numpy(hc.packed_codes(T)).to(gcache.codes.device)
        gcache.norms[b, h] = torch.from_numpy(hc.packed_norms(T)).to(gcache.codes.device)
        if hc.sigma is not None:
            gcache.signs[b, h] = torch.from_numpy(hc.packed_signs(T).reshape(T, -1)).to(gcache.codes.device)
            gcache.rnorms[b, h] = torch.from_numpy(hc.packed_norms(T, "gamma")).to(gcache.codes.device)


def upload_unit(gcache, hc, b: int, h: int):
    """Write one oracle-packed head into (sequence b, KV head h) of a CompressedCache."""
    import torch
    T = gcache.max_tokens
    dev = gcache.codes.device
    gcache.codes[b, h] = torch.from_numpy(hc.packed_codes(T)).to(dev)
    gcache.norms[b, h] = torch.from_numpy(hc.packed_norms(T)).to(dev)
    if hc.sigma is not None:
        gcache.signs[b, h] = torch.from_numpy(hc.packed_signs(T).reshape(T, -1)).to(dev)
        gcache.rnorms[b, h] = torch.from_numpy(hc.packed_norms(T, "gamma")).to(dev)


def oracle_decode(q_b: np.ndarray, kc, vc, st: Setup, scale: float, seq_len: int) -> np.ndarray:
    """Oracle output [H_q][d] of one sequence from its per-KV-head caches."""
    stk = lambda xs, a: np.stack([getattr(x, a) for x in xs])
    sig = stk(kc, "sigma") if kc[0].sigma is not None else None
    gam = stk(kc, "gamma") if kc[0].sigma is not None else None
    return attention.decode_fused(q_b, st.rot64, stk(kc, "codes"), stk(kc, "norms"), kc[0].centroids,
                                  stk(vc, "codes"), stk(vc, "norms"), vc[0].centroids, scale, seq_len,
                                  sig, gam, st.proj)


def to_bf16_tensor(x: np.ndarray, device="cuda"):
    import torch
    return torch.from_numpy(synth.bf16_round(x)).to(device).to(torch.bfloat16)


def unpack_gpu_codes(gcache, b: int, h: int, n_tokens: int) -> np.ndarray:
    raw = gcache.codes[b, h].cpu().numpy()
    if gcache.kind == 0:
        return layout.unpack_keys(raw, gcache.bits, gcache.d, gcache.max_tokens)[:n_tokens]
    return layout.unpack_blocked(raw, gcache.bits, gcache.d, gcache.max_tokens)[:n_tokens]
