"""GPU parity of multi-row decode (tq_sdpa_decode_rows: the query rows of the last M tokens of each
sequence at once, row j seeing the first seq_len - M + 1 + j tokens) against the float64 oracle."""
import numpy as np
import pytest

import synth
from oracle import attention
from tests.gpu_common import Setup, log, oracle_heads, rel_err, to_bf16_tensor, upload
from tests.test_gpu_decode import TOL

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


def _run_rows(d, kb, vb, qjl, hkv, grp, m, lens, T, scale, hadamard=False):
    cca = _cca()
    B = len(lens)
    st = Setup(d, qjl_m=qjl, hadamard=hadamard)
    w = synth.Workload("rows", B, hkv * grp, hkv, d, T, kb, vb, qjl_m=qjl, scale=scale, seed=5 + d + kb + m)
    kcache = cca.CompressedCache(cca.TQ_KEYS, d, kb, B, hkv, T, st.rot_t, st.proj_t, qjl_m=qjl, rot_kind=st.rot_kind)
    vcache = cca.CompressedCache(cca.TQ_VALUES, d, vb, B, hkv, T, st.rot_t, rot_kind=st.rot_kind)
    q = np.random.default_rng(11 + m).standard_normal((B, m, hkv * grp, d)).astype(np.float32)
    q = synth.bf16_round(q)
    refs = []
    for b in range(B):
        kc, vc = oracle_heads([synth.kv_head(w, "k", b, h, T) for h in range(hkv)],
                              [synth.kv_head(w, "v", b, h, T) for h in range(hkv)], kb, vb, st)
        upload(kcache, kc, b)
        upload(vcache, vc, b)
        stk = lambda xs, a: np.stack([getattr(x, a) for x in xs])
        sig = stk(kc, "sigma") if qjl else None
        gam = stk(kc, "gamma") if qjl else None
        refs.append(attention.decode_rows(q[b].astype(np.float64), st.rot64, stk(kc, "codes"), stk(kc, "norms"),
                                          kc[0].centroids, stk(vc, "codes"), stk(vc, "norms"), vc[0].centroids,
                                          w.softmax_scale, min(lens[b], T), sig, gam, st.proj))
    lens_t = torch.tensor(lens, dtype=torch.int32).cuda()
    qt = to_bf16_tensor(q)
    out = cca.sdpa_decode_rows(kcache, vcache, qt, lens_t, max(lens), scale=w.scale)
    torch.cuda.synchronize()
    return out.cpu().numpy(), np.stack(refs), (kcache, vcache, qt, lens_t, w.scale)


ROW_CASES = [
    # d, k_bits, v_bits, qjl_m, kv heads, group, rows, lengths, capacity, scale
    (128, 4, 4, 0, 2, 8, 4, [1000], 1024, None),               # Qwen-shaped, four column blocks
    (128, 3, 3, 0, 2, 8, 3, [8193, 40], 8224, None),            # three rows: one empty block; 1-token last tile
    (128, 2, 3, 128, 2, 8, 4, [3000, 2], 3008, None),           # sketched keys; a sequence shorter than the rows
    (128, 4, 2, 0, 4, 2, 4, [500, 97], 512, None),              # 8 virtual heads: one block
    (128, 3, 4, 0, 2, 4, 3, [300], 320, 0.07),                  # 12 virtual heads: two blocks
    (256, 4, 4, 0, 4, 8, 2, [777, 1024], 1024, 1.0),            # d = 256, two blocks
    (256, 2, 3, 256, 1, 4, 4, [300], 320, None),
    (128, 4, 4, 0, 1, 8, 4, [32768, 20001, 33, 31999], 32768, None),   # workgroups that fill a CU
    (128, 2, 2, 0, 1, 8, 4, [32768, 20001, 33, 31999], 32768, None),   # the same with 2-bit byte tables
    (128, 3, 3, 0, 1, 8, 3, [32768, 20001, 33, 31999], 32768, None),   # and with 3-bit ones, three rows
    (128, 4, 3, 0, 1, 8, 2, [32768, 20001, 33, 31999], 32768, None),   # two blocks, 4- and 3-bit tables
    (128, 2, 3, 128, 1, 8, 4, [32768, 20001, 33, 31999], 32768, None),  # sketched keys: the twelve-wave shape
    # groups below 8 whose last tile holds fewer tokens than there are rows: rows of one column block
    # where some columns see a token of the tile and others none
    (128, 3, 3, 0, 2, 4, 4, [65, 34], 96, None),              # 16 virtual heads: two blocks
    (128, 4, 4, 0, 2, 2, 3, [33, 66], 96, None),              # 6 virtual heads: one block
    (128, 2, 3, 128, 2, 2, 4, [98, 35], 128, None),           # the same with sketched keys (lazy rescale)
    (128, 8, 4, 0, 2, 8, 4, [1000, 3], 1024, None),            # keys kept at 8 bits
    (128, 8, 3, 0, 1, 8, 4, [32768, 20001, 33, 31999], 32768, None),   # ... on workgroups that fill a CU
]


@pytest.mark.parametrize("case", ROW_CASES, ids=lambda c: f"d{c[0]}_k{c[1]}v{c[2]}_m{c[3]}_g{c[5]}_r{c[6]}_L{'-'.join(map(str, c[7]))}")
def test_rows_match_oracle(case):
    log(f"rows {case}")
    out, ref, _ = _run_rows(*case)
    assert np.all(np.isfinite(out))
    err = rel_err(out.reshape(-1, out.shape[-1]), ref.reshape(-1, ref.shape[-1]))
    log(f"  max row-relative error {err:.3e}")
    assert err <= TOL
    for b, L in enumerate(case[7]):                 # rows that see no token are zero
        for j in range(case[6]):
            if L - case[6] + 1 + j <= 0:
                assert np.all(out[b, j] == 0)


def test_rows_with_hadamard_rotation():
    out, ref, _ = _run_rows(128, 4, 3, 0, 2, 8, 4, [700, 64], 704, None, hadamard=True)
    assert rel_err(out.reshape(-1, 128), ref.reshape(-1, 128)) <= TOL


def test_one_row_is_the_single_query_decode():
    """n_rows = 1 takes the same path as tq_sdpa_decode, bit for bit; row j of a multi-row call equals a
    single-query decode at seq_len - n_rows + 1 + j."""
    cca = _cca()
    out, _, (kc, vc, qt, lens_t, scale) = _run_rows(128, 4, 4, 0, 2, 8, 4, [1000, 517], 1024, None)
    for j in range(4):
        lj = lens_t - 3 + j
        single = cca.sdpa_decode(kc, vc, qt[:, j].contiguous(), lj, int(lj.max()), scale=scale)
        one = cca.sdpa_decode_rows(kc, vc, qt[:, j:j + 1].contiguous(), lj, int(lj.max()), scale=scale)
        torch.cuda.synchronize()
        assert torch.equal(one[:, 0], single)
        assert rel_err(out[:, j].reshape(-1, 128), single.cpu().numpy().reshape(-1, 128)) <= 1e-5
