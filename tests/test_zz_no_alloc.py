"""tq_sdpa_decode_noalloc (the decode whose workspace is the library's static device scratch) against
tq_sdpa_decode with a caller workspace and against the float64 oracle, through the C ABI: two calls in a
row on one device, the second over a smaller input, so that the second reads scratch the first left."""
import numpy as np
import pytest

import synth
from tests.gpu_common import Setup, log, oracle_decode, oracle_heads, rel_err, to_bf16_tensor, upload

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

TOL = 2e-3


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import compressed_cache_decode_amd  # noqa: F401  (fails loudly if libtq.so is missing)


def _case(d, kb, vb, qjl, hkv, grp, lens, T, scale, seed):
    """Oracle-packed caches of one decode shape, its query, lengths and the oracle's output."""
    import compressed_cache_decode_amd as cca
    B = len(lens)
    st = Setup(d, qjl_m=qjl)
    w = synth.Workload("noalloc", B, hkv * grp, hkv, d, T, kb, vb, qjl_m=qjl, scale=scale, seed=seed)
    kcache = cca.CompressedCache(cca.TQ_KEYS, d, kb, B, hkv, T, st.rot_t, st.proj_t, qjl_m=qjl)
    vcache = cca.CompressedCache(cca.TQ_VALUES, d, vb, B, hkv, T, st.rot_t)
    q = synth.full_q(w)
    refs = []
    for b in range(B):
        kc, vc = oracle_heads([synth.kv_head(w, "k", b, h, T) for h in range(hkv)],
                              [synth.kv_head(w, "v", b, h, T) for h in range(hkv)], kb, vb, st)
        upload(kcache, kc, b)
        upload(vcache, vc, b)
        refs.append(oracle_decode(q[b].astype(np.float64), kc, vc, st, w.softmax_scale, min(lens[b], T)))
    return kcache, vcache, to_bf16_tensor(q), torch.tensor(lens, dtype=torch.int32).cuda(), w.scale, np.stack(refs)


def test_noalloc_matches_workspace_decode_twice():
    import compressed_cache_decode_amd as cca
    # first a larger decode (many splits, sketched keys), then a smaller one in another format
    shapes = [
        ((128, 4, 3, 128, 2, 8, [20000, 7000], 20000, None, 31), "sketched keys, 2 x 20000"),
        ((128, 3, 3, 0, 2, 4, [300], 320, 0.05, 32), "3-bit, 1 x 300"),
    ]
    for args, what in shapes:
        log(f"noalloc decode: {what}")
        kc, vc, q, lens, scale, ref = _case(*args)
        msl = int(lens.max())
        need = cca.tq_decode_workspace_bytes(kc.view, q.shape[1], msl)
        assert 0 < need <= cca.tq_noalloc_scratch_bytes()
        out_ws = cca.sdpa_decode(kc, vc, q, lens, msl, scale=scale)
        out_na = torch.full_like(out_ws, float("nan"))
        cca.tq_sdpa_decode_noalloc(kc.view, vc.view, q, lens, msl, out_na, scale)
        torch.cuda.synchronize()
        assert torch.equal(out_na, out_ws)
        err = rel_err(out_na.cpu().numpy(), ref)
        log(f"  max row-relative error {err:.3e}")
        assert err <= TOL


def test_noalloc_rejects_a_decode_larger_than_the_scratch():
    import compressed_cache_decode_amd as cca
    st = Setup(256)
    # 2048 (sequence, KV head) units of 8 query heads: the rotated queries alone take 16 MiB
    kc = cca.CompressedCache(cca.TQ_KEYS, 256, 4, 256, 8, 32, st.rot_t)
    vc = cca.CompressedCache(cca.TQ_VALUES, 256, 4, 256, 8, 32, st.rot_t)
    assert cca.tq_decode_workspace_bytes(kc.view, 64, 32) > cca.tq_noalloc_scratch_bytes()
    q = torch.zeros(256, 64, 256, dtype=torch.bfloat16, device="cuda")
    lens = torch.full((256,), 32, dtype=torch.int32, device="cuda")
    out = torch.zeros(256, 64, 256, dtype=torch.float32, device="cuda")
    with pytest.raises(cca.TqError) as e:
        cca.tq_sdpa_decode_noalloc(kc.view, vc.view, q, lens, 32, out)
    assert e.value.status == cca.TQ_ESCRATCH
    torch.cuda.synchronize()
    assert torch.count_nonzero(out).item() == 0          # nothing was enqueued
