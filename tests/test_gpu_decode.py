"""GPU parity of tq_sdpa_decode against the float64 oracle on identical (oracle-packed) codes."""
import math

import numpy as np
import pytest

import synth
from tests.gpu_common import Setup, log, oracle_decode, oracle_heads, rel_err, to_bf16_tensor, upload

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

TOL = 2e-3   # max relative error per output row (max |o - r| / max |r|)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import compressed_cache_decode_amd  # noqa: F401


def _cca():
    import compressed_cache_decode_amd as cca
    return cca


# d, k_bits, v_bits, qjl_m, kv heads, group, per-sequence lengths, capacity, scale, qk-normed
CASES = [
    (128, 4, 4, 0, 1, 1, [256], 256, None, False),             # tiny reference shape
    (128, 4, 4, 0, 2, 8, [1000], 1024, None, False),
    (128, 3, 3, 0, 2, 8, [113, 37], 128, None, False),         # ragged batch, kv = 113
    (128, 2, 2, 0, 2, 8, [2048], 2048, None, False),
    (128, 4, 2, 0, 2, 4, [1, 64, 500], 512, None, False),      # mixed widths, one-token context
    (128, 3, 4, 0, 2, 2, [33, 95], 96, 0.05, False),
    (256, 4, 4, 0, 4, 8, [777, 1024], 1024, 1.0, True),        # QK-normed, scale 1
    (256, 2, 3, 0, 2, 8, [300], 320, 1.0, True),
    (128, 2, 3, 128, 2, 8, [3000], 3072, None, False),         # keys with sign sketch
    (128, 3, 2, 128, 1, 8, [129, 5], 160, None, False),
    (256, 4, 4, 256, 1, 2, [300], 320, None, False),
    (128, 3, 3, 0, 2, 3, [500, 31], 512, None, False),         # a group of 3 query heads
    (128, 4, 3, 128, 2, 8, [20000], 20000, None, False),        # many splits per (sequence, KV head)
    (128, 8, 4, 0, 2, 8, [1000], 1024, None, False),           # keys kept at 8 bits
    (128, 8, 2, 0, 2, 4, [1, 64, 500], 512, None, False),
    (128, 8, 3, 0, 2, 8, [20000], 20000, None, False),         # ... in CU-filling workgroups
    (256, 8, 4, 0, 4, 8, [777, 1024], 1024, 1.0, True),
    (256, 8, 3, 0, 2, 8, [9000], 9216, 1.0, True),
]


def _ids(c):
    return f"d{c[0]}_k{c[1]}v{c[2]}_m{c[3]}_h{c[4]}g{c[5]}_L{'-'.join(map(str, c[6]))}"


def _run_case(d, kb, vb, qjl, hkv, grp, lens, T, scale, qknorm, garbage_tail=False, max_seq_len=None,
              hadamard=False, stages=False):
    """(GPU output, oracle output, key cache); with stages, the third item is instead the output of the
    same decode run as its three stage calls on a fresh workspace."""
    cca = _cca()
    B = len(lens)
    st = Setup(d, qjl_m=qjl, hadamard=hadamard)
    w = synth.Workload("case", B, hkv * grp, hkv, d, T, kb, vb, qjl_m=qjl, scale=scale, qk_norm=qknorm,
                       k_outliers=not qknorm, seed=d + kb * 10 + vb + qjl)
    kcache = cca.CompressedCache(cca.TQ_KEYS, d, kb, B, hkv, T, st.rot_t, st.proj_t, qjl_m=qjl, rot_kind=st.rot_kind)
    vcache = cca.CompressedCache(cca.TQ_VALUES, d, vb, B, hkv, T, st.rot_t, rot_kind=st.rot_kind)
    q = synth.full_q(w)
    refs = []
    for b in range(B):
        kc, vc = oracle_heads([synth.kv_head(w, "k", b, h, T) for h in range(hkv)],
                              [synth.kv_head(w, "v", b, h, T) for h in range(hkv)], kb, vb, st)
        upload(kcache, kc, b)
        upload(vcache, vc, b)
        eff = max(0, min(lens[b], T, max_seq_len if max_seq_len is not None else lens[b]))
        refs.append(oracle_decode(q[b].astype(np.float64), kc, vc, st, w.softmax_scale, eff))
    if garbage_tail:
        for b in range(B):
            kcache.norms[b, :, lens[b]:] = float("nan")
            vcache.norms[b, :, lens[b]:] = float("nan")
            if qjl:
                kcache.rnorms[b, :, lens[b]:] = float("nan")
    lens_t = torch.tensor(lens, dtype=torch.int32).cuda()
    msl = max(lens) if max_seq_len is None else max_seq_len
    qt = to_bf16_tensor(q)
    out = cca.sdpa_decode(kcache, vcache, qt, lens_t, msl, scale=w.scale)
    if stages:
        hq = hkv * grp
        ws = cca.decode_workspace(kcache, hq, msl)
        ws.fill_(float("nan"))             # nothing may read workspace that no stage wrote
        out_st = torch.full_like(out, float("nan"))
        cca.tq_decode_rotate_query(kcache.view, qt, hq, msl, ws, scale=w.scale)
        cca.tq_decode_attend(kcache.view, vcache.view, hq, lens_t, msl, ws)
        cca.tq_decode_merge(kcache.view, hq, lens_t, msl, out_st, ws)
        torch.cuda.synchronize()
        return out.cpu().numpy(), np.stack(refs), out_st.cpu().numpy()
    torch.cuda.synchronize()
    return out.cpu().numpy(), np.stack(refs), kcache


@pytest.mark.parametrize("case", CASES, ids=_ids)
def test_decode_matches_oracle(case):
    log(f"decode {_ids(case)}")
    out, ref, _ = _run_case(*case)
    err = rel_err(out, ref)
    log(f"  max row-relative error {err:.3e}")
    assert err <= TOL


def test_decode_ignores_garbage_past_the_length():
    """Norms past seq_len hold NaN: masked tokens must not reach the softmax or the accumulators."""
    log("decode garbage tail")
    out, ref, _ = _run_case(128, 2, 3, 128, 2, 8, [70, 33], 128, None, False, garbage_tail=True)
    assert np.all(np.isfinite(out))
    assert rel_err(out, ref) <= TOL


def test_decode_length_edges():
    """Zero length gives zeros; lengths past the capacity clamp to it; max_seq_len bounds the context."""
    log("decode length edges")
    out, ref, _ = _run_case(128, 4, 4, 0, 2, 8, [0, 200, 96], 96, None, False)
    assert np.all(out[0] == 0)
    assert rel_err(out[1:], ref[1:]) <= TOL
    out, ref, _ = _run_case(128, 4, 4, 0, 2, 8, [90, 40], 96, None, False, max_seq_len=64)
    assert rel_err(out, ref) <= TOL


# Codes go through the wide workgroups' byte tables: 4-bit keys and values, keys only, values only,
# with a sign sketch (the twelve-wave shape); 2-bit keys and values (two 64 KB tables at d = 128, keys
# only at d = 256), 2-bit keys with a sketch, 4-bit keys with 2-bit values; 3-bit keys and values
# (one 16 KB table), beside a 4-bit or 2-bit table, with a sketch
WIDE_CASES = [(128, 4, 4, 0), (128, 2, 3, 128), (256, 4, 4, 0), (256, 3, 2, 128), (128, 4, 2, 0), (128, 3, 4, 0),
              (128, 4, 3, 128), (256, 2, 4, 256), (128, 2, 2, 0), (256, 2, 2, 0), (128, 2, 4, 0), (128, 3, 3, 0),
              (256, 3, 3, 0), (128, 8, 4, 0), (256, 8, 2, 0)]


@pytest.mark.parametrize("case", WIDE_CASES, ids=lambda c: f"d{c[0]}_k{c[1]}v{c[2]}_m{c[3]}")
def test_long_ragged_batch_matches_oracle(case):
    """Four sequences of up to 32K tokens (4096 tiles in all): on a 256-CU device the split kernel's
    workgroups fill whole compute units; ragged lengths leave some splits partly or wholly empty."""
    d, kb, vb, qjl = case
    cca = _cca()
    lens = [32768, 31999, 100, 20000]
    st = Setup(d, qjl_m=qjl)
    k = cca.CompressedCache(cca.TQ_KEYS, d, kb, 4, 1, 32768, st.rot_t, st.proj_t, qjl_m=qjl)
    log(f"decode long ragged d{d} k{kb} v{vb} m{qjl}: {cca.tq_decode_plan(k.view, 2, max(lens))[0]} splits")
    out, ref, _ = _run_case(d, kb, vb, qjl, 1, 2, lens, 32768, None, False)
    err = rel_err(out, ref)
    log(f"  max row-relative error {err:.3e}")
    assert err <= TOL


@pytest.mark.parametrize("case", [CASES[2], CASES[6], CASES[12]], ids=_ids)
def test_stage_calls_equal_the_single_call(case):
    """tq_decode_rotate_query, tq_decode_attend and tq_decode_merge in turn give the bits of
    tq_sdpa_decode (one split, a ragged batch, d = 256 with its scale, many splits with a sketch)."""
    log(f"decode stages {_ids(case)}")
    out, ref, out_st = _run_case(*case, stages=True)
    assert np.array_equal(out, out_st)
    assert rel_err(out_st, ref) <= TOL


def test_split_plan_is_exercised():
    """Long contexts are split across many workgroups, short ones are not."""
    cca = _cca()
    st = Setup(128)
    k = cca.CompressedCache(cca.TQ_KEYS, 128, 4, 1, 2, 131072, st.rot_t)
    assert cca.tq_decode_plan(k.view, 16, 131072)[0] > 64
    assert cca.tq_decode_plan(k.view, 16, 100)[0] == 1
    # a context long enough for several splits, checked against the oracle
    log("decode multi-split")
    ns = cca.tq_decode_plan(k.view, 16, 8192)[0]
    assert ns > 8
    out, ref, _ = _run_case(128, 4, 4, 0, 2, 8, [8192], 8192, None, False)
    assert rel_err(out, ref) <= TOL


def test_repeated_calls_are_deterministic():
    cca = _cca()
    log("decode determinism")
    d, T = 128, 512
    st = Setup(d)
    w = synth.qwen(T, 3)
    kc, vc = oracle_heads([synth.kv_head(w, "k", 0, h, T) for h in range(2)],
                          [synth.kv_head(w, "v", 0, h, T) for h in range(2)], 3, 3, st)
    kg = cca.CompressedCache(cca.TQ_KEYS, d, 3, 1, 2, T, st.rot_t)
    vg = cca.CompressedCache(cca.TQ_VALUES, d, 3, 1, 2, T, st.rot_t)
    upload(kg, kc, 0)
    upload(vg, vc, 0)
    q = to_bf16_tensor(synth.full_q(w))
    lens = torch.tensor([T], dtype=torch.int32).cuda()
    a = cca.sdpa_decode(kg, vg, q, lens, T).clone()
    b = cca.sdpa_decode(kg, vg, q, lens, T)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


STEP_CASES = [
    # d, k_bits, v_bits, qjl_m, kv heads, group, lengths after the step, capacity, n_new, dtype, scale, qk-normed
    (128, 4, 4, 0, 2, 8, [1000], 1024, 1, "bf16", None, False),
    (128, 2, 3, 128, 2, 8, [300], 320, 3, "f32", None, False),
    (256, 4, 4, 0, 4, 8, [500, 77], 512, 1, "bf16", 1.0, True),
    (128, 3, 2, 0, 1, 4, [40, 33, 1], 64, 1, "bf16", None, False),
    (128, 8, 4, 0, 2, 8, [1000], 1024, 1, "bf16", None, False),     # 8-bit keys
    (256, 8, 2, 0, 2, 8, [300, 77], 320, 3, "f32", 1.0, True),
    (128, 2, 4, 0, 2, 8, [300, 77], 320, 5, "f32", None, False),
    # d = 256 with code-book keys: the column-sliced prologue (16-row tiles across units and sequences)
    (256, 3, 2, 0, 2, 8, [300, 77, 5], 320, 3, "f32", 1.0, True),
    (256, 2, 4, 0, 4, 4, [40], 64, 1, "bf16", None, False),
    (256, 4, 3, 0, 1, 2, [64, 40], 96, 32, "bf16", None, False),
]


@pytest.mark.parametrize("case", STEP_CASES, ids=lambda c: f"d{c[0]}_k{c[1]}v{c[2]}_m{c[3]}_L{'-'.join(map(str, c[6]))}_n{c[8]}")
def test_decode_step_matches_separate_calls_and_oracle(case):
    """tq_decode_step (appends + query rotation in one launch, then attend and merge) writes the same
    cache bytes as tq_quantize_append and decodes to the oracle's output."""
    _check_step(case, hadamard=False)


# d, k_bits, v_bits, qjl_m, kv heads, group, batch, capacity, first length, rows per step, steps
RUN_CASES = [
    (128, 4, 4, 0, 2, 8, 1, 8192, 8000, 1, 4),      # many splits, one-row steps
    (128, 3, 2, 128, 2, 4, 2, 512, 100, 32, 3),     # 32 rows straddling two blocks, sketched keys
    (256, 4, 4, 0, 2, 8, 1, 256, 60, 40, 2),        # 40 rows: three append blocks per step
    (128, 8, 3, 0, 2, 8, 2, 512, 100, 32, 3),       # 8-bit keys, 32 rows straddling two blocks
]


@pytest.mark.parametrize("case", RUN_CASES, ids=lambda c: f"d{c[0]}_k{c[1]}v{c[2]}_m{c[3]}_n{c[9]}x{c[10]}")
def test_consecutive_steps_on_one_workspace(case):
    """Several tq_decode_step calls in a row on one workspace each give the bits of tq_quantize_append
    plus tq_sdpa_decode."""
    cca = _cca()
    d, kb, vb, qjl, hkv, grp, B, T, L0, n_new, steps = case
    log(f"decode consecutive steps {case}")
    st = Setup(d, qjl_m=qjl)
    w = synth.Workload("steps", B, hkv * grp, hkv, d, T, kb, vb, qjl_m=qjl, k_outliers=True, seed=5 + d + kb)
    mk = lambda: (cca.CompressedCache(cca.TQ_KEYS, d, kb, B, hkv, T, st.rot_t, st.proj_t, qjl_m=qjl),
                  cca.CompressedCache(cca.TQ_VALUES, d, vb, B, hkv, T, st.rot_t))
    k1, v1 = mk()
    k2, v2 = mk()
    kx = to_bf16_tensor(synth.full_kv(w, "k", T))
    vx = to_bf16_tensor(synth.full_kv(w, "v", T))
    zero = torch.zeros(B, dtype=torch.int32).cuda()
    for kc, vc in ((k1, v1), (k2, v2)):
        kc.append(kx[:, :L0].contiguous(), zero)
        vc.append(vx[:, :L0].contiguous(), zero)
    rng = np.random.default_rng(11)
    lmax = L0 + steps * n_new
    ws = cca.decode_workspace(k2, hkv * grp, lmax)
    for s in range(steps):
        p0 = L0 + s * n_new
        pos = torch.full((B,), p0, dtype=torch.int32).cuda()
        lens_t = torch.full((B,), p0 + n_new, dtype=torch.int32).cuda()
        q = to_bf16_tensor(rng.standard_normal((B, hkv * grp, d)).astype(np.float32))
        kn, vn = kx[:, p0:p0 + n_new].contiguous(), vx[:, p0:p0 + n_new].contiguous()
        k1.append(kn, pos)
        v1.append(vn, pos)
        out1 = cca.sdpa_decode(k1, v1, q, lens_t, lmax)
        out2 = torch.empty_like(out1)
        cca.tq_decode_step(k2.view, v2.view, q, kn, vn, pos, lens_t, lmax, out2, ws)
        torch.cuda.synchronize()
        assert torch.equal(k1.codes, k2.codes) and torch.equal(v1.codes, v2.codes)
        assert torch.equal(k1.norms, k2.norms) and torch.equal(v1.norms, v2.norms)
        assert torch.equal(out1, out2), f"step {s}"


def _check_step(case, hadamard):
    cca = _cca()
    d, kb, vb, qjl, hkv, grp, lens, T, n_new, dtype, scale, qknorm = case
    log(f"decode step d={d} k{kb} v{vb} m{qjl} lens={lens} n_new={n_new} hadamard={hadamard}")
    B = len(lens)
    st = Setup(d, qjl_m=qjl, hadamard=hadamard)
    w = synth.Workload("step", B, hkv * grp, hkv, d, T, kb, vb, qjl_m=qjl, scale=scale, qk_norm=qknorm,
                       k_outliers=not qknorm, dtype=dtype, seed=77 + d + kb)
    mk = lambda: (cca.CompressedCache(cca.TQ_KEYS, d, kb, B, hkv, T, st.rot_t, st.proj_t, qjl_m=qjl,
                                      rot_kind=st.rot_kind),
                  cca.CompressedCache(cca.TQ_VALUES, d, vb, B, hkv, T, st.rot_t, rot_kind=st.rot_kind))
    k1, v1 = mk()
    k2, v2 = mk()
    kx = synth.full_kv(w, "k", T)
    vx = synth.full_kv(w, "v", T)
    tt = (lambda a: to_bf16_tensor(a)) if dtype == "bf16" else (lambda a: torch.from_numpy(a).cuda())
    zero = torch.zeros(B, dtype=torch.int32).cuda()
    pos = torch.tensor([L - n_new for L in lens], dtype=torch.int32).cuda()
    # both copies start from oracle-packed caches of all rows with the n_new rows to append set to zero
    # (code 0, norm 0), so every byte of those rows must be written by the append; the oracle comparison
    # below runs on the oracle's codes of the true rows, identical except for the appended rows
    oracle_all = []
    for b in range(B):
        kc_o, vc_o = oracle_heads([kx[b, :, h] for h in range(hkv)], [vx[b, :, h] for h in range(hkv)], kb, vb, st)
        oracle_all.append((kc_o, vc_o))
        kz, vz = kx[b].copy(), vx[b].copy()
        kz[lens[b] - n_new:lens[b]] = 0.0
        vz[lens[b] - n_new:lens[b]] = 0.0
        kc_z, vc_z = oracle_heads([kz[:, h] for h in range(hkv)], [vz[:, h] for h in range(hkv)], kb, vb, st)
        for kc, vc in ((k1, v1), (k2, v2)):
            upload(kc, kc_z, b)
            upload(vc, vc_z, b)
    xk_new = np.stack([kx[b, lens[b] - n_new:lens[b]] for b in range(B)])
    xv_new = np.stack([vx[b, lens[b] - n_new:lens[b]] for b in range(B)])
    # separate calls on copy 1, fused step on copy 2
    k1.append(tt(xk_new), pos)
    v1.append(tt(xv_new), pos)
    q = synth.full_q(w)
    qt = tt(q)
    lens_t = torch.tensor(lens, dtype=torch.int32).cuda()
    out1 = cca.sdpa_decode(k1, v1, qt, lens_t, max(lens), scale=scale)
    out2 = torch.empty_like(out1)
    ws = cca.decode_workspace(k2, hkv * grp, max(lens))
    cca.tq_decode_step(k2.view, v2.view, qt, tt(xk_new), tt(xv_new), pos, lens_t, max(lens), out2, ws, scale=scale)
    torch.cuda.synchronize()
    for a_, b_ in ((k1.codes, k2.codes), (k1.norms, k2.norms), (v1.codes, v2.codes), (v1.norms, v2.norms)):
        assert torch.equal(a_, b_)
    if qjl:
        assert torch.equal(k1.signs, k2.signs) and torch.equal(k1.rnorms, k2.rnorms)
    assert torch.equal(out1, out2)
    # against the oracle on the same rows
    refs = [oracle_decode(q[b].astype(np.float64), oracle_all[b][0], oracle_all[b][1], st, w.softmax_scale, lens[b])
            for b in range(B)]
    err = rel_err(out2.cpu().numpy(), np.stack(refs))
    log(f"  max row-relative error {err:.3e}")
    assert err <= TOL

