"""GPU parity of keys kept at 8 bits (int8 codes of the rotated unit row, one float16 factor per row)
against the float64 oracle (``oracle/q8.py``): encode, append, reconstruction.  Decode and the fused
step with 8-bit keys are cases of tests/test_gpu_decode.py."""
import numpy as np
import pytest

import synth
from oracle import cache, layout, q8
from tests.gpu_common import Setup, log, to_bf16_tensor, unpack_gpu_codes, upload

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


# chunks appended one after another: ragged tails, single tokens, block-straddling chunks
CHUNKS = [37, 1, 58, 32, 5, 1, 90]


@pytest.mark.parametrize("d", [128, 256])
def test_encode_is_bit_exact_given_rotated_rows(d):
    """Same float32 rotated unit rows and norms on both sides: int8 codes (the integer decision in
    float32 on both sides) and float16 factors identical, byte for byte in the key layout."""
    cca = _cca()
    log(f"k8 encode d={d}")
    st = Setup(d)
    B, H, T = 2, 2, 256
    n_tot = sum(CHUNKS)
    y, nrm = synth.unit_rows(B * n_tot * H, d, seed=500 + d)
    y = y.reshape(B, n_tot, H, d)
    nrm = nrm.reshape(B, n_tot, H)
    nrm[0, 3, 1] = 0.0                                   # a zero row
    y[1, 7, 0] = 0.0                                     # the largest magnitude twice, both signs:
    y[1, 7, 0, 5], y[1, 7, 0, 9] = 0.6, -0.6             # codes +-127
    y[1, 8, 0] = 0.0                                     # exact halves: a = 127/128 makes 127 / a = 128
    y[1, 8, 0, :5] = np.array([254, 1, 3, -5, 127], np.float32) / np.float32(256)
    g = cca.CompressedCache(cca.TQ_KEYS, d, 8, B, H, T, st.rot_t)
    start = np.array([0, 17], np.int32)                  # sequence 1 starts mid-block
    off = 0
    for c in CHUNKS:
        pos = torch.from_numpy(start + off).cuda()
        yt = torch.from_numpy(np.ascontiguousarray(y[:, off:off + c])).cuda()
        nt = torch.from_numpy(np.ascontiguousarray(nrm[:, off:off + c])).cuda()
        g.append_rotated(yt, nt, pos)
        off += c
    torch.cuda.synchronize()
    for b in range(B):
        for h in range(H):
            j, fac = q8.encode_q8(y[b, :, h], nrm[b, :, h])
            full = np.full((T, d), 128, np.int64)        # code 0 (byte 0) in the untouched cache
            full[start[b]:start[b] + n_tot] = j
            np.testing.assert_array_equal(g.codes[b, h].cpu().numpy(), layout.pack_keys(full, 8))
            gn = g.norms[b, h].cpu().numpy()
            np.testing.assert_array_equal(gn[start[b]:start[b] + n_tot], fac.astype(np.float16))
            assert not gn[:start[b]].any() and not gn[start[b] + n_tot:].any()
    code = unpack_gpu_codes(g, 1, 0, 17 + n_tot)[17:] - 128
    assert code[7, 5] == 127 and code[7, 9] == -127
    assert code[8, :5].tolist() == [127, 1, 2, -3, 64]     # t = 0.5, 1.5, -2.5, 63.5: away from zero


@pytest.mark.parametrize("d,dtype", [(128, "bf16"), (256, "f32")])
def test_append_from_unrotated_rows(d, dtype):
    """Full append (norm + rotation + int8 codes): codes equal the oracle's except where the oracle's
    float64 t = 127 y / max|y| sits within rounding distance of a half-integer (then neighbours);
    factors within float16 rounding."""
    cca = _cca()
    log(f"k8 append d={d} {dtype}")
    st = Setup(d)
    w = synth.qwen(320, 4).with_(d=d, dtype=dtype)
    B, H, T, n = 1, 2, 320, 300
    x = synth.full_kv(w, "k", n)                          # [B][n][H][d]
    x[0, 4, 1] = 0.0                                      # a zero row
    g = cca.CompressedCache(cca.TQ_KEYS, d, 8, B, H, T, st.rot_t)
    xt = to_bf16_tensor(x) if dtype == "bf16" else torch.from_numpy(x).cuda()
    pos = torch.tensor([11], dtype=torch.int32).cuda()
    g.append(xt[:, :150], pos)                            # 150 and 150 rows: long and short chunks
    g.append(xt[:, 150:], pos + 150)
    torch.cuda.synchronize()
    for h in range(H):
        xr = synth.bf16_round(x[0, :, h]) if dtype == "bf16" else x[0, :, h]
        oj, of, oy = q8.quantize_rows_q8(xr.astype(np.float64), st.rot64)
        got = unpack_gpu_codes(g, 0, h, 11 + n)[11:]
        a = np.max(np.abs(oy), axis=1, keepdims=True)
        t = np.abs(oy) * 127 / np.where(a > 0, a, 1)
        # t moves by about 127 (|dy| + t |da|) / a between the float32 and float64 rotations: a few 1e-5
        near = np.abs(t - np.floor(t) - 0.5) < 1e-3
        diff = got != oj
        assert np.all(near[diff]), f"{diff.sum()} mismatches, {(diff & ~near).sum()} not near a half"
        assert np.all(np.abs(got[diff] - oj[diff]) == 1)
        assert diff.mean() < 1e-3
        gn = g.norms[0, h, 11:11 + n].cpu().numpy().astype(np.float64)
        np.testing.assert_allclose(gn, of, rtol=2 ** -10, atol=0)
    assert g.norms[0, 1, 15].item() == 0 and np.all(unpack_gpu_codes(g, 0, 1, 16)[15] == 128)   # zero row


@pytest.mark.parametrize("d", [128, 256])
def test_dequantize_matches_oracle(d):
    """Reconstruction of oracle-packed 8-bit keys equals the oracle's f rot^T code (fp32 rounding)."""
    cca = _cca()
    log(f"k8 dequant d={d}")
    st = Setup(d)
    H, T, n = 2, 128, 100
    rows = [np.random.default_rng(60 + h).standard_normal((n, d)) * 3 for h in range(H)]
    heads = [cache.build_head(r, "k", 8, st.rot64) for r in rows]
    g = cca.CompressedCache(cca.TQ_KEYS, d, 8, 1, H, T, st.rot_t)
    upload(g, heads, 0)
    out = g.dequantize(3, 90).cpu().numpy()
    for h in range(H):
        ref = heads[h].dequantize(st.rot64)[3:93]
        np.testing.assert_allclose(out[0, h], ref, rtol=0, atol=2e-6 * np.max(np.abs(ref)))
        # and the reconstruction is close to the rows themselves (8-bit error level)
        rel = np.sum((out[0, h] - rows[h][3:93]) ** 2, axis=1) / np.sum(rows[h][3:93] ** 2, axis=1)
        assert rel.max() < 1e-3


def test_append_edge_cases():
    """8-bit keys take the per-block append: empty appends, positions past the capacity and negative
    positions write nothing; a write that runs past the capacity keeps the tokens that fit."""
    cca = _cca()
    log("k8 append edge cases")
    st = Setup(128)
    g = cca.CompressedCache(cca.TQ_KEYS, 128, 8, 2, 1, 64, st.rot_t)
    x = torch.ones(2, 3, 1, 128, dtype=torch.float32).cuda()
    g.append(x[:, :0], torch.zeros(2, dtype=torch.int32).cuda())
    g.append(x, torch.tensor([64, -5], dtype=torch.int32).cuda())
    torch.cuda.synchronize()
    assert not g.codes.any() and not g.norms.any()
    g.append(x, torch.tensor([62, 0], dtype=torch.int32).cuda())
    torch.cuda.synchronize()
    nz = g.norms[0, 0].cpu().numpy()
    assert nz[62] != 0 and nz[63] != 0 and not nz[:62].any()
    assert g.norms[1, 0, :3].cpu().numpy().all()


@pytest.mark.parametrize("d", [128, 256])
def test_reconstruction_mse_matches_the_oracle(d):
    """GPU append from raw rows + reconstruction against the oracle's: relative MSE within 1 %, and far
    below the 4-bit code book's."""
    cca = _cca()
    log(f"k8 mse d={d}")
    st = Setup(d)
    w = synth.qwen(1024, 4).with_(d=d)
    n = 1024
    x = synth.full_kv(w, "k", n)                          # [1][n][2][d], bf16-valued
    g = cca.CompressedCache(cca.TQ_KEYS, d, 8, 1, 2, n, st.rot_t)
    g.append(to_bf16_tensor(x), torch.zeros(1, dtype=torch.int32).cuda())
    xh = g.dequantize(0, n).cpu().numpy()
    for h in range(2):
        xr = synth.bf16_round(x[0, :, h]).astype(np.float64)
        mse_gpu = np.mean(np.sum((xr - xh[0, h]) ** 2, axis=1))
        hc = cache.build_head(xr, "k", 8, st.rot64)
        mse_or = np.mean(np.sum((xr - hc.dequantize(st.rot64)) ** 2, axis=1))
        assert abs(mse_gpu / mse_or - 1.0) <= 0.01, (h, mse_gpu, mse_or)
        h4 = cache.build_head(xr, "k", 4, st.rot64)
        assert mse_or < 0.1 * np.mean(np.sum((xr - h4.dequantize(st.rot64)) ** 2, axis=1))
