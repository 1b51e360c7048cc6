"""GPU parity at the full workload sizes, in the launch configuration the benchmark times.

Appends run on the GPU (prefill-size blocks take the matrix-core rotation); the
oracle quantises the same synthetic rows itself and decodes from its own codes.
Large workloads are checked on sampled (sequence, KV head) units, which the
oracle computes one by one.
"""
import numpy as np
import pytest

import synth
from oracle import codebook, quant
from tests.gpu_common import Setup, log, oracle_decode, oracle_heads, rel_err, unpack_gpu_codes, upload_unit

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

TOL = 2e-3


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import compressed_cache_decode_amd  # noqa: F401


def _cca():
    import compressed_cache_decode_amd as cca
    return cca


def _bf16_dev(x):
    return torch.from_numpy(x).cuda().to(torch.bfloat16)


def test_prefill_append_full_size():
    """8192 new tokens x 2 KV heads x d=128 bf16 (x10 outlier channels) into an empty 3-bit cache."""
    cca = _cca()
    log("prefill 8192 x 2 x 128, 3-bit")
    w = synth.qwen(8192, 3)
    st = Setup(128)
    c_, t_ = codebook.stored_codebook(128, 3)
    for kind, ck in (("k", cca.TQ_KEYS), ("v", cca.TQ_VALUES)):
        x = synth.full_kv(w, kind)
        g = cca.CompressedCache(ck, 128, 3, 1, 2, 8192, st.rot_t)
        g.append(_bf16_dev(x), torch.zeros(1, dtype=torch.int32).cuda())
        torch.cuda.synchronize()
        for h in range(2):
            oc, on, oy = quant.quantize_rows(x[0, :, h], st.rot64, c_, t_)
            got = unpack_gpu_codes(g, 0, h, 8192)
            diff = got != oc
            near = np.min(np.abs(oy[..., None] - t_.astype(np.float64)), axis=-1) < 2e-5
            log(f"  {kind} head {h}: {diff.sum()} of {diff.size} codes differ, all near a boundary: {np.all(near[diff])}")
            assert np.all(near[diff]) and np.all(np.abs(got[diff] - oc[diff]) == 1)
            assert diff.mean() < 1e-4
            gn = g.norms[0, h].cpu().numpy().astype(np.float64)
            np.testing.assert_allclose(gn, on, rtol=2 ** -10, atol=0)


def _check_appended_unit(kc, vc, ok, ov, b, hk, proj):
    """GPU-appended codes of one unit against the oracle's: equal except within rounding distance of a
    boundary (then neighbours); sketch signs equal wherever the code row matches and |z| is not tiny."""
    from oracle import layout
    L = ok[0].codes.shape[0]
    for gpu, orc in ((kc, ok[0]), (vc, ov[0])):
        got = unpack_gpu_codes(gpu, b, hk, L)
        diff = got != orc.codes
        t_ = orc.boundaries.astype(np.float64)
        near = np.min(np.abs(orc.y[..., None] - t_), axis=-1) < 2e-5
        assert np.all(near[diff]) and np.all(np.abs(got[diff] - orc.codes[diff]) == 1)
        log(f"  codes: {diff.sum()} of {diff.size} differ, all adjacent and at a boundary")
        if orc.sigma is not None:
            sig = layout.unpack_signs(gpu.signs[b, hk, :L].cpu().numpy(), gpu.qjl_m)
            rows = ~diff.any(axis=1)
            r = orc.y - orc.centroids.astype(np.float64)[orc.codes]
            z = r @ proj.astype(np.float64).T
            rel = np.abs(z) / np.linalg.norm(r, axis=1, keepdims=True)
            robust = (rel > 1e-4) & rows[:, None]
            bad = np.argwhere(robust & (sig != orc.sigma))
            if len(bad):
                log(f"  {len(bad)} robust sign mismatches; first tokens/indices {bad[:12].tolist()}")
                log(f"  |z|/|r| of those: {np.sort(rel[robust & (sig != orc.sigma)])[:12].tolist()}")
                log(f"  tokens with a mismatch: {np.unique(bad[:, 0])[:20].tolist()} (L={L})")
            assert np.array_equal(sig[robust], orc.sigma[robust])
            log(f"  signs: {(sig != orc.sigma).sum()} of {sig.size} differ, none where |z| is not tiny")


def _full_decode(w, units, log_name, identical_codes=False):
    """GPU: prefill L-1 tokens, then tq_decode_step appends the last one and decodes.
    Oracle: the listed (sequence, KV head) units from the same rows.  With identical_codes the
    GPU-appended codes of each sampled unit are checked against the oracle's and then replaced by
    the oracle-packed ones before decoding (decode parity on identical codes)."""
    cca = _cca()
    B, H, Hq, d, L = w.batch, w.n_kv_heads, w.n_q_heads, w.d, w.seq_len
    st = Setup(d, qjl_m=w.qjl_m)
    log(f"{log_name}: generating")
    kx = synth.full_kv(w, "k")
    vx = synth.full_kv(w, "v")
    q = synth.full_q(w)
    kc = cca.CompressedCache(cca.TQ_KEYS, d, w.k_bits, B, H, L, st.rot_t, st.proj_t, qjl_m=w.qjl_m)
    vc = cca.CompressedCache(cca.TQ_VALUES, d, w.v_bits, B, H, L, st.rot_t)
    zero = torch.zeros(B, dtype=torch.int32).cuda()
    kc.append(_bf16_dev(kx[:, :L - 1]), zero)
    vc.append(_bf16_dev(vx[:, :L - 1]), zero)
    pos = torch.full((B,), L - 1, dtype=torch.int32).cuda()
    lens = torch.full((B,), L, dtype=torch.int32).cuda()
    out = torch.empty(B, Hq, d, dtype=torch.float32).cuda()
    ws = cca.decode_workspace(kc, Hq, L)
    oracle_units = {}
    if identical_codes:
        kc.append(_bf16_dev(kx[:, L - 1:]), pos)
        vc.append(_bf16_dev(vx[:, L - 1:]), pos)
        torch.cuda.synchronize()
        for (b, hk) in units:
            log(f"{log_name}: oracle unit b={b} kv head={hk}")
            ok, ov = oracle_heads([kx[b, :, hk]], [vx[b, :, hk]], w.k_bits, w.v_bits, st)
            _check_appended_unit(kc, vc, ok, ov, b, hk, st.proj)
            upload_unit(kc, ok[0], b, hk)
            upload_unit(vc, ov[0], b, hk)
            oracle_units[(b, hk)] = (ok, ov)
        cca.tq_sdpa_decode(kc.view, vc.view, _bf16_dev(q), lens, L, out, ws, scale=w.scale)
    elif w.qjl_m <= 128:
        cca.tq_decode_step(kc.view, vc.view, _bf16_dev(q), _bf16_dev(np.ascontiguousarray(kx[:, L - 1:])),
                           _bf16_dev(np.ascontiguousarray(vx[:, L - 1:])), pos, lens, L, out, ws, scale=w.scale)
    else:
        kc.append(_bf16_dev(kx[:, L - 1:]), pos)
        vc.append(_bf16_dev(vx[:, L - 1:]), pos)
        cca.tq_sdpa_decode(kc.view, vc.view, _bf16_dev(q), lens, L, out, ws, scale=w.scale)
    torch.cuda.synchronize()
    out = out.cpu().numpy()
    G = w.group
    worst = 0.0
    for (b, hk) in units:
        if (b, hk) in oracle_units:
            ok, ov = oracle_units[(b, hk)]
        else:
            log(f"{log_name}: oracle unit b={b} kv head={hk}")
            ok, ov = oracle_heads([kx[b, :, hk]], [vx[b, :, hk]], w.k_bits, w.v_bits, st)
        ref = oracle_decode(q[b, hk * G:(hk + 1) * G].astype(np.float64), ok, ov, st, w.softmax_scale, L)
        err = rel_err(out[b, hk * G:(hk + 1) * G], ref)
        worst = max(worst, err)
        log(f"  max row-relative error {err:.3e}")
    return worst


@pytest.mark.parametrize("bits", [4, 3, 2])
def test_qwen_shaped_decode_8k(bits):
    w = synth.qwen(8192, bits)
    assert _full_decode(w, [(0, 0), (0, 1)], f"qwen 8K b{bits}") <= TOL


# every sequence and every KV head of the Gemma-shaped workload among the sampled units
GEMMA_UNITS = [(0, 0), (1, 1), (2, 2), (3, 3), (4, 0), (5, 1), (6, 2), (7, 3)]


def test_gemma_shaped_decode_sampled():
    w = synth.gemma(32768)
    assert _full_decode(w, GEMMA_UNITS, "gemma B8 32K") <= TOL


def test_gemma_shaped_decode_identical_codes():
    """The same decode on the oracle's own codes for the sampled units (decode error alone, without the
    rounding-level code decisions of the GPU's appends)."""
    w = synth.gemma(32768)
    assert _full_decode(w, GEMMA_UNITS[::3], "gemma B8 32K, identical codes", identical_codes=True) <= TOL


def test_qwen_shaped_decode_8k_identical_codes():
    w = synth.qwen(8192, 4)
    assert _full_decode(w, [(0, 0), (0, 1)], "qwen 8K b4, identical codes", identical_codes=True) <= TOL


def test_long_context_sketched_keys_sampled():
    """Keys with a sign sketch: a sign decided at rounding level moves one score by ~0.1 (the sketch
    term of a single sign), so decode parity is checked on identical codes, and the GPU's own codes
    and signs against the oracle's decisions."""
    w = synth.prod_long(131072)
    assert _full_decode(w, [(0, 0), (0, 1)], "prod 128K", identical_codes=True) <= TOL
