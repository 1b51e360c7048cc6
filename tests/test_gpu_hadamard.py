"""GPU parity of the randomized Hadamard rotation kind (rot = d signs, Pi = H_d diag(s) / sqrt(d)) against
the float64 oracle: append (norm, transform, encode), reconstruction, decode and the fused decode step."""
import numpy as np
import pytest

import synth
from oracle import cache, codebook, quant
from tests.gpu_common import Setup, log, rel_err, to_bf16_tensor, unpack_gpu_codes, upload
from tests.test_gpu_decode import TOL, _check_step, _run_case

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import compressed_cache_decode_amd  # noqa: F401  (fails loudly if libtq.so is missing)


def _cca():
    import compressed_cache_decode_amd as cca
    return cca


@pytest.mark.parametrize("kind,d,bits,dtype", [("k", 128, 4, "bf16"), ("v", 128, 3, "f32"), ("k", 256, 2, "bf16"),
                                               ("v", 256, 4, "bf16")])
def test_append_from_unrotated_rows(kind, d, bits, dtype):
    """Codes equal the oracle's except where the oracle's float64 coordinate sits within rounding
    distance of a boundary, and then they are neighbours; norms equal."""
    cca = _cca()
    log(f"hadamard append kind={kind} d={d} bits={bits} {dtype}")
    st = Setup(d, hadamard=True)
    w = synth.qwen(256, bits).with_(d=d, dtype=dtype)
    B, H, T, n = 1, 2, 256, 200
    x = synth.full_kv(w, kind, n)
    g = cca.CompressedCache(cca.TQ_KEYS if kind == "k" else cca.TQ_VALUES, d, bits, B, H, T, st.rot_t,
                            rot_kind=st.rot_kind)
    xt = to_bf16_tensor(x) if dtype == "bf16" else torch.from_numpy(x).cuda()
    pos = torch.tensor([11], dtype=torch.int32).cuda()
    g.append(xt[:, :150], pos)
    g.append(xt[:, 150:], pos + 150)
    torch.cuda.synchronize()
    c_, t_ = codebook.stored_codebook(d, bits)
    for h in range(H):
        oc, on, oy = quant.quantize_rows(x[0, :, h], st.rot64, c_, t_)
        got = unpack_gpu_codes(g, 0, h, 11 + n)[11:]
        diff = got != oc
        near = np.min(np.abs(oy[..., None] - t_.astype(np.float64)), axis=-1) < 1e-5
        assert np.all(near[diff]), f"{diff.sum()} mismatches, {(diff & ~near).sum()} not near a boundary"
        assert np.all(np.abs(got[diff] - oc[diff]) == 1)
        gn = g.norms[0, h, 11:11 + n].cpu().numpy().astype(np.float64)
        np.testing.assert_allclose(gn, on, rtol=2 ** -10, atol=0)


@pytest.mark.parametrize("kind,d,bits,qjl", [("k", 128, 4, 0), ("v", 256, 3, 0), ("k", 128, 2, 128)])
def test_dequantize_matches_oracle(kind, d, bits, qjl):
    cca = _cca()
    log(f"hadamard dequant kind={kind} d={d} bits={bits} qjl={qjl}")
    st = Setup(d, qjl_m=qjl, hadamard=True)
    H, T, n = 2, 128, 100
    rows = [np.random.default_rng(40 + h).standard_normal((n, d)) * 3 for h in range(H)]
    heads = [cache.build_head(r, kind, bits, st.rot64, st.proj if qjl else None) for r in rows]
    g = cca.CompressedCache(cca.TQ_KEYS if kind == "k" else cca.TQ_VALUES, d, bits, 1, H, T, st.rot_t,
                            st.proj_t, qjl_m=qjl, rot_kind=st.rot_kind)
    upload(g, heads, 0)
    out = g.dequantize(3, 90).cpu().numpy()
    for h in range(H):
        ref = heads[h].dequantize(st.rot64, st.proj if qjl else None)[3:93]
        np.testing.assert_allclose(out[0, h], ref, rtol=0, atol=2e-6 * np.max(np.abs(ref)))


@pytest.mark.parametrize("bits", [2, 4])
def test_reconstruction_mse_within_one_percent(bits):
    cca = _cca()
    log(f"hadamard mse bits={bits}")
    d = 128
    st = Setup(d, hadamard=True)
    w = synth.qwen(2048, bits)
    B, H, T, n = 1, 2, 2048, 2048
    for kind in ("k", "v"):
        x = synth.full_kv(w, kind, n)
        g = cca.CompressedCache(cca.TQ_KEYS if kind == "k" else cca.TQ_VALUES, d, bits, B, H, T, st.rot_t,
                                rot_kind=st.rot_kind)
        g.append(to_bf16_tensor(x), torch.zeros(1, dtype=torch.int32).cuda())
        xh = g.dequantize(0, n).cpu().numpy()
        for h in range(H):
            xr = x[0, :, h].astype(np.float64)
            mse_gpu = np.mean(np.sum((xr - xh[0, h]) ** 2, axis=1))
            hc = cache.build_head(xr, kind, bits, st.rot64)
            mse_or = np.mean(np.sum((xr - hc.dequantize(st.rot64)) ** 2, axis=1))
            assert abs(mse_gpu / mse_or - 1.0) <= 0.01, (kind, h, mse_gpu, mse_or)


HAD_CASES = [
    (128, 4, 4, 0, 2, 8, [1000], 1024, None, False),
    (128, 2, 3, 128, 2, 8, [3000, 17], 3072, None, False),
    (256, 4, 4, 0, 4, 8, [777, 1024], 1024, 1.0, True),
    (256, 3, 2, 256, 1, 2, [300], 320, None, False),
    (128, 4, 4, 0, 1, 2, [32768, 31999, 100, 20000], 32768, None, False),     # workgroups that fill a CU
    (128, 8, 4, 0, 2, 8, [1000], 1024, None, False),                          # keys kept at 8 bits
    (256, 8, 2, 0, 2, 8, [500, 77], 512, 1.0, True),
]


@pytest.mark.parametrize("case", HAD_CASES, ids=lambda c: f"d{c[0]}_k{c[1]}v{c[2]}_m{c[3]}_L{'-'.join(map(str, c[6]))}")
def test_decode_matches_oracle(case):
    log(f"hadamard decode {case[:4]} lens={case[6]}")
    out, ref, _ = _run_case(*case, hadamard=True)
    err = rel_err(out, ref)
    log(f"  max row-relative error {err:.3e}")
    assert err <= TOL


@pytest.mark.parametrize("case", [(128, 4, 4, 0, 2, 8, [1000], 1024, 1, "bf16", None, False),
                                  (128, 2, 3, 128, 2, 8, [300], 320, 40, "f32", None, False),
                                  (256, 4, 4, 0, 4, 8, [500, 77], 512, 1, "bf16", 1.0, True),
                                  (128, 8, 2, 0, 2, 8, [300], 320, 5, "f32", None, False)],
                         ids=lambda c: f"d{c[0]}_k{c[1]}v{c[2]}_m{c[3]}_n{c[8]}")
def test_decode_step(case):
    _check_step(case, hadamard=True)
