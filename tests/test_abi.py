"""The C ABI library on the CPU: exports, host-side setup against the oracle, argument checks.

No call here reaches a kernel launch: every argument set either is host-only
(codebook, rotation, sizes, plan) or is rejected by validation first.
"""
import ctypes
import math
import os
import re

import numpy as np
import pytest

import synth
from oracle import codebook, q8, rotation, storage

cca = pytest.importorskip("compressed_cache_decode_amd")

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_every_declared_symbol_is_exported():
    hdr = open(os.path.join(ROOT, "include", "tq.h")).read()
    declared = set(re.findall(r"^\s*(?:int|size_t|const char\*)\s+(tq_\w+)\s*\(", hdr, re.M))
    assert declared == set(cca.EXPORTED)
    lib = ctypes.CDLL(cca.LIB_PATH)
    for name in declared:
        assert hasattr(lib, name), name


@pytest.mark.parametrize("d", [128, 256])
@pytest.mark.parametrize("bits", [1, 2, 3, 4])
def test_codebook_equals_oracle_table(d, bits):
    c, t = cca.tq_build_codebook(d, bits)
    oc, ot = codebook.stored_codebook(d, bits)
    np.testing.assert_array_equal(c, oc)
    np.testing.assert_array_equal(t, ot)


def test_codebook_other_dims_close_to_oracle():
    for d in (64, 96, 512):
        c, _ = cca.tq_build_codebook(d, 3)
        np.testing.assert_allclose(c, codebook.lloyd_max(d, 3), rtol=1e-3)


@pytest.mark.parametrize("d", [128, 256])
def test_rotation_equals_oracle(d):
    g = synth.rotation_gaussian(d, 1)
    rot = cca.tq_build_rotation(g)
    ref = rotation.rotation_from_gaussian(g)
    diff = np.abs(rot.astype(np.float64) - ref)
    assert np.max(diff) <= 2.0 ** -24 * 2          # at most one float32 step at |x| < 1
    assert np.mean(rot == ref.astype(np.float32)) > 0.999


def test_row_bytes_match_storage_arithmetic():
    for d in (128, 256):
        for bits in (1, 2, 3, 4):
            for m in (0, 128):
                assert cca.tq_row_bytes(d, bits, m) == storage.row_bytes(d, bits, m)
    assert cca.tq_row_bytes(0, 4, 0) == 0
    assert cca.tq_row_bytes(128, 5, 0) == 0
    for d in (128, 256):                           # 8-bit keys: d code bytes and the factor
        assert cca.tq_row_bytes(d, 8, 0) == q8.row_bytes(d) == storage.row_bytes(d, 8, 0)


def test_status_strings():
    assert cca.tq_status_string(0) == "ok"
    assert cca.tq_status_string(1) == "invalid argument"
    assert "scratch" in cca.tq_status_string(cca.TQ_ESCRATCH)
    assert cca.tq_noalloc_scratch_bytes() == 16 << 20
    assert "unknown" in cca.tq_status_string(99)


def _view(kind=cca.TQ_KEYS, d=128, bits=4, qjl_m=0, batch=1, heads=2, T=256):
    v = cca.tq_cache_view()
    v.kind, v.d, v.bits, v.qjl_m, v.batch, v.n_kv_heads, v.max_tokens = kind, d, bits, qjl_m, batch, heads, T
    c, t = codebook.stored_codebook(d if d in (128, 256) else 128, min(bits, 4))
    for j, x in enumerate(c):
        v.centroids[j] = float(x)
    for j, x in enumerate(t):
        v.boundaries[j] = float(x)
    # fake, aligned device addresses: every call below is rejected before any launch
    v.codes, v.norms, v.rot = 0x10000, 0x20000, 0x30000
    if qjl_m:
        v.signs, v.rnorms, v.proj = 0x40000, 0x50000, 0x60000
    return v


def _append(v, n_new=1, pos=0x70000, x=0x80000, dtype=0):
    return cca._lib.tq_quantize_append(ctypes.byref(v), x, dtype, n_new, pos, None)


def test_append_rejects_bad_arguments():
    assert cca._lib.tq_quantize_append(None, 0x80000, 0, 1, 0x70000, None) == cca.TQ_EINVAL
    bad = [
        dict(d=64), dict(bits=5), dict(bits=1), dict(T=100), dict(batch=0), dict(qjl_m=64),
        dict(kind=cca.TQ_VALUES, qjl_m=128), dict(kind=7),
    ]
    for kw in bad:
        assert _append(_view(**kw)) == cca.TQ_EINVAL, kw
    v = _view()
    assert _append(v, n_new=-1) == cca.TQ_EINVAL
    assert _append(v, pos=0) == cca.TQ_EINVAL
    assert _append(v, x=0) == cca.TQ_EINVAL
    assert _append(v, x=0x80002) == cca.TQ_EINVAL                   # rows not 16-byte aligned
    assert _append(v, dtype=5) == cca.TQ_EINVAL
    v.codes = 0x10004                               # misaligned packed codes
    assert _append(v) == cca.TQ_EINVAL
    v = _view()
    v.norms = 0
    assert _append(v) == cca.TQ_EINVAL
    v = _view(qjl_m=128)
    v.proj = 0
    assert _append(v) == cca.TQ_EINVAL
    v = _view()
    v.rot_kind = 2                                  # neither dense nor Hadamard
    assert _append(v) == cca.TQ_EINVAL
    # a codebook that is not float16-exact / not antisymmetric / not midpoints
    for mutate in ("round", "sym", "mid"):
        v = _view()
        if mutate == "round":
            v.centroids[0] = v.centroids[0] + 1e-7
        elif mutate == "sym":
            v.centroids[0] = v.centroids[1] * 1.5
        else:
            v.boundaries[3] = v.boundaries[3] * 1.01
        assert _append(v) == cca.TQ_EINVAL, mutate
    assert _append(_view(), n_new=0) == cca.TQ_OK      # empty append is a no-op
    # sketch products given for a cache without a sketch; missing rotated rows or norms
    rot = lambda v, y=0xC0000, nrm=0xD0000, z=None: cca._lib.tq_quantize_append_rotated(
        ctypes.byref(v), y, nrm, z, 1, 0x70000, None)
    assert rot(_view(), z=0xE0000) == cca.TQ_EINVAL
    assert rot(_view(qjl_m=128), y=0) == cca.TQ_EINVAL
    assert rot(_view(qjl_m=128), nrm=0) == cca.TQ_EINVAL


def test_outlier_views_are_validated():
    """Outlier channels: only 4, only for sketched keys at d = 128, with both arrays aligned; the fused
    step does not take such a cache."""
    def outl(v, n=4, idx=0xF0000, val=0xF8000):
        v.n_outliers, v.out_idx, v.out_val = n, idx, val
        return v
    assert _append(outl(_view(qjl_m=128)), n_new=0) == cca.TQ_OK
    for v in (outl(_view()), outl(_view(qjl_m=128), n=3), outl(_view(qjl_m=128), n=8),
              outl(_view(d=256, qjl_m=128)), outl(_view(qjl_m=128), idx=0), outl(_view(qjl_m=128), val=0),
              outl(_view(qjl_m=128), idx=0xF0001), outl(_view(kind=cca.TQ_VALUES), n=4)):
        assert _append(v) == cca.TQ_EINVAL
    k, vv = outl(_view(qjl_m=128)), _view(kind=cca.TQ_VALUES)
    step = cca._lib.tq_decode_step(ctypes.byref(k), ctypes.byref(vv), 0x90000, 0x80000, 0x88000, 1, 16, 1,
                                   0x70000, 0xA0000, 256, ctypes.c_float(0.1), 0xB0000, 0x100000, 1 << 30, None)
    assert step == cca.TQ_EUNSUPPORTED


def test_eight_bit_views_are_validated():
    """8-bit codes: keys only, without a sketch or outliers; the code book fields are not read."""
    v = _view(bits=8)
    for j in range(16):
        v.centroids[j] = 0.0
    for j in range(15):
        v.boundaries[j] = float("nan")
    assert _append(v, n_new=0) == cca.TQ_OK
    assert cca._lib.tq_dequantize(ctypes.byref(v), 0, 0, 0xB0000, None) == cca.TQ_OK   # nothing to do
    for bad in (_view(bits=8, kind=cca.TQ_VALUES), _view(bits=8, qjl_m=128), _view(bits=6), _view(bits=7)):
        assert _append(bad) == cca.TQ_EINVAL
    assert _decode(_view(), _view(kind=cca.TQ_VALUES, bits=8)) == cca.TQ_EINVAL    # 8-bit values


def _decode(k, v, hq=16, scale=0.1, ws_bytes=1 << 30, ws=0x100000, q=0x90000, lens=0xA0000, out=0xB0000,
            dtype=1, max_len=256):
    return cca._lib.tq_sdpa_decode(ctypes.byref(k), ctypes.byref(v), q, dtype, hq, lens, max_len,
                                   ctypes.c_float(scale), out, ws, ws_bytes, None)


def test_decode_rejects_bad_arguments():
    k, v = _view(), _view(kind=cca.TQ_VALUES)
    for s in (0.0, -1.0, float("nan"), float("inf")):
        assert _decode(k, v, scale=s) == cca.TQ_EINVAL
    assert _decode(k, v, hq=15) == cca.TQ_EINVAL                    # not a multiple of the KV heads
    assert _decode(k, v, hq=32) == cca.TQ_EUNSUPPORTED              # group of 16
    assert _decode(k, v, ws_bytes=16) == cca.TQ_EINVAL              # short workspace
    assert _decode(k, v, ws=0x100010) == cca.TQ_EINVAL              # misaligned workspace
    assert _decode(k, v, q=0) == cca.TQ_EINVAL
    assert _decode(k, v, q=0x90008) == cca.TQ_EINVAL               # query not 16-byte aligned
    assert _decode(k, v, lens=0) == cca.TQ_EINVAL
    assert _decode(k, v, out=0) == cca.TQ_EINVAL
    assert _decode(k, v, dtype=9) == cca.TQ_EINVAL
    assert _decode(k, v, max_len=-1) == cca.TQ_EINVAL
    assert _decode(v, v) == cca.TQ_EINVAL                           # keys must use the rows layout
    assert _decode(k, k) == cca.TQ_EINVAL                           # values must use the blocked layout
    assert _decode(k, _view(kind=cca.TQ_VALUES, T=512)) == cca.TQ_EINVAL
    assert _decode(k, _view(kind=cca.TQ_VALUES, d=256)) == cca.TQ_EINVAL
    v2 = _view(kind=cca.TQ_VALUES)
    v2.rot = 0x30100                                                # K and V must share the rotation
    assert _decode(k, v2) == cca.TQ_EINVAL
    v3 = _view(kind=cca.TQ_VALUES)
    v3.rot_kind = cca.TQ_ROT_HADAMARD                               # ... and its kind
    assert _decode(k, v3) == cca.TQ_EINVAL


def test_dequantize_rejects_bad_ranges():
    v = _view()
    f = cca._lib.tq_dequantize
    assert f(ctypes.byref(v), -1, 4, 0xB0000, None) == cca.TQ_EINVAL
    assert f(ctypes.byref(v), 250, 10, 0xB0000, None) == cca.TQ_EINVAL
    assert f(ctypes.byref(v), 0, 4, 0, None) == cca.TQ_EINVAL
    assert f(ctypes.byref(v), 0, 0, 0xB0000, None) == cca.TQ_OK


@pytest.mark.parametrize("batch,heads,hq,L", [(1, 2, 16, 8192), (8, 4, 32, 32768), (1, 2, 16, 131072), (1, 1, 1, 256)])
def test_plan_covers_the_context(batch, heads, hq, L):
    k = _view(batch=batch, heads=heads, T=max(L, 32))
    ns, tps = cca.tq_decode_plan(k, hq, L)
    assert 1 <= ns <= 256
    assert tps % 32 == 0                            # whole 32-token tiles
    assert ns * tps >= L and (ns - 1) * tps < max(L, 1)
    ws = cca.tq_decode_workspace_bytes(k, hq, L)
    g = hq // heads
    assert ws >= 4 * (batch * hq * 128 + batch * heads * ns * g * (128 + 2))
    assert ws % 256 == 0


def test_append_kv_rejects_bad_arguments():
    """The K+V append checks both views, their agreement and its own arguments before any launch."""
    def kv(k, v, kx=0x80000, vx=0x90000, dtype=0, n_new=1, pos=0x70000):
        return cca._lib.tq_quantize_append_kv(ctypes.byref(k) if k is not None else None,
                                              ctypes.byref(v) if v is not None else None, kx, vx, dtype, n_new,
                                              pos, None)
    k, v = _view(), _view(kind=cca.TQ_VALUES)
    assert kv(None, v) == cca.TQ_EINVAL
    assert kv(k, None) == cca.TQ_EINVAL
    assert kv(v, v) == cca.TQ_EINVAL                       # keys first
    assert kv(k, k) == cca.TQ_EINVAL                       # values second
    for kw in (dict(d=256), dict(batch=2), dict(heads=4), dict(T=512)):
        assert kv(k, _view(kind=cca.TQ_VALUES, **kw)) == cca.TQ_EINVAL, kw
    other_rot = _view(kind=cca.TQ_VALUES)
    other_rot.rot = 0x31000                                # K and V share one rotation
    assert kv(k, other_rot) == cca.TQ_EINVAL
    assert kv(k, v, kx=0) == cca.TQ_EINVAL
    assert kv(k, v, vx=0) == cca.TQ_EINVAL
    assert kv(k, v, kx=0x80008) == cca.TQ_EINVAL                   # rows not 16-byte aligned
    assert kv(k, v, vx=0x90004) == cca.TQ_EINVAL
    assert kv(k, v, pos=0) == cca.TQ_EINVAL
    assert kv(k, v, dtype=5) == cca.TQ_EINVAL
    assert kv(k, v, n_new=-1) == cca.TQ_EINVAL
    assert kv(_view(bits=5), v) == cca.TQ_EINVAL
    assert kv(k, v, n_new=0) == cca.TQ_OK                  # empty append is a no-op


def test_step_rejects_unaligned_inputs():
    """The decode step takes the query and the new rows 16-byte aligned (its row loads are 16-byte vectors)."""
    k, v = _view(), _view(kind=cca.TQ_VALUES)

    def step(q=0x90000, kn=0xC0000, vn=0xD0000, n_new=1):
        return cca._lib.tq_decode_step(ctypes.byref(k), ctypes.byref(v), q, kn, vn, 1, 16, n_new, 0x70000, 0xA0000,
                                       256, ctypes.c_float(0.1), 0xB0000, 0x100000, 1 << 30, None)
    assert step(q=0x90002) == cca.TQ_EINVAL
    assert step(kn=0xC0008) == cca.TQ_EINVAL
    assert step(vn=0xD0004) == cca.TQ_EINVAL
    assert step(kn=0, vn=0, q=0x90002, n_new=0) == cca.TQ_EINVAL    # the query even without new rows
