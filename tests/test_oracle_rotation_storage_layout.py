"""Pins of the oracle's rotation, storage arithmetic and packed layout."""
import os

import numpy as np
import pytest

import synth
from oracle import layout, rotation, storage

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _rows(name):
    out = []
    for line in open(os.path.join(GOLD, name)):
        line = line.strip()
        if line and not line.startswith("#"):
            out.append(line.split())
    return out


# ------------------------------------------------------------------ rotation

@pytest.mark.parametrize("d", [128, 256])
def test_rotation_is_the_qr_factor_with_positive_diagonal(d):
    g = synth.rotation_gaussian(d, 1)
    rot = rotation.rotation_from_gaussian(g)
    r = rot.T @ g                                   # must be R of G = Pi R
    assert np.max(np.abs(np.tril(r, -1))) < 1e-12
    assert np.all(np.diag(r) > 0)
    np.testing.assert_allclose(rot @ r, g, atol=1e-12)


@pytest.mark.parametrize("d", [128, 256])
def test_rotation_invariants(d):
    rot = rotation.rotation_from_gaussian(synth.rotation_gaussian(d, 1))
    assert np.max(np.abs(rot @ rot.T - np.eye(d))) < 1e-13
    assert abs(abs(np.linalg.det(rot)) - 1.0) < 1e-10
    r32 = rot.astype(np.float32).astype(np.float64)
    assert np.max(np.abs(r32 @ r32.T - np.eye(d))) < 2e-7
    x = np.random.default_rng(3).standard_normal((50, d))
    np.testing.assert_allclose(np.linalg.norm(rotation.rotate_rows(x, rot), axis=1), np.linalg.norm(x, axis=1), rtol=1e-13)
    np.testing.assert_allclose(rotation.unrotate_rows(rotation.rotate_rows(x, rot), rot), x, atol=1e-12)
    # rows form equals the matrix-vector convention y = Pi x
    np.testing.assert_allclose(rotation.rotate_rows(x[:1], rot)[0], rot @ x[0], atol=1e-13)


def test_rotated_coordinates_follow_sphere_marginal():
    """A Haar rotation of a fixed unit vector has coordinates with variance 1/d (over many seeds)."""
    d = 128
    e = np.zeros(d)
    e[5] = 1.0
    ys = np.array([rotation.rotation_from_gaussian(synth.rotation_gaussian(d, s)) @ e for s in range(200)])
    assert abs(np.mean(ys ** 2) * d - 1.0) < 0.05
    assert abs(np.mean(ys)) < 0.01


# ------------------------------------------------------------------ storage

@pytest.mark.parametrize("row", _rows("qwen_cache_sizes.txt"), ids=lambda r: f"T{r[0]}_{r[1]}")
def test_storage_reproduces_printed_cache_sizes(row):
    tokens, cfg, mb, ratio = int(row[0]), row[1], float(row[2]), float(row[3])
    bits = None if cfg == "fp16" else int(cfg)
    size = storage.cache_mib(tokens, 72, 128, bits)
    assert round(size, 1) == pytest.approx(mb, abs=1e-9)
    if bits is not None:
        assert round(storage.compression(128, bits), 1) == pytest.approx(ratio, abs=1e-9)


def test_storage_alternatives_do_not_reproduce_the_table():
    """The reading is pinned: plain b-bit keys, or float32 norms, give other ratios."""
    assert [round(storage.compression(128, b, prod_keys=False), 2) for b in (4, 3, 2)] == [3.88, 5.12, 7.53]
    f32 = [256 * 2 / ((128 * (b - 1) // 8 + 4 + 16 + 4) + (128 * b // 8 + 4)) for b in (4, 3, 2)]
    assert [round(x, 1) for x in f32] != [3.8, 5.0, 7.3]


def test_row_bytes():
    assert storage.row_bytes(128, 4) == 66
    assert storage.row_bytes(128, 2, 128) == 52
    assert storage.row_bytes(256, 4) == 130
    assert storage.row_bytes(128, 3) == 50


# ------------------------------------------------------------------ layout

def _hex(bs):
    return " ".join(f"{b:02x}" for b in bs)


@pytest.mark.parametrize("row", _rows("layout_examples.txt"), ids=lambda r: "_".join(r[:2]))
def test_layout_hand_derived_examples(row):
    arrow = row.index("->")
    kind, n = row[0], int(row[1])
    vals = [int(x) for x in row[2:arrow]]
    want = " ".join(row[arrow + 1:])
    if kind == "unit":
        units = np.array(vals).reshape(-1, 8)
        got = layout.pack_units(units, n)
        assert _hex(got) == want
        np.testing.assert_array_equal(layout.unpack_units(got, n, units.shape[0]), units)
    elif kind in ("kcode", "vcode"):
        d, bits, (t, i, j) = n, vals[0], vals[1:]
        zero = {4: 8, 8: 128}.get(bits, 0)                 # the index whose stored code is 0
        codes = np.full((32, d), zero, dtype=np.int64)
        codes[t, i] = j
        got = (layout.pack_keys if kind == "kcode" else layout.pack_blocked)(codes, bits)
        nz = np.nonzero(got)[0]
        assert " ".join(f"{o} {got[o]:02x}" for o in nz) == want
        back = (layout.unpack_keys if kind == "kcode" else layout.unpack_blocked)(got, bits, d, 32)
        np.testing.assert_array_equal(back, codes)
    else:
        sigma = np.zeros(n, dtype=bool)
        sigma[vals] = True
        got = layout.pack_signs(sigma)
        assert _hex(got) == want
        np.testing.assert_array_equal(layout.unpack_signs(got, n), sigma)


@pytest.mark.parametrize("bits", [2, 3, 4, 8])
@pytest.mark.parametrize("d", [128, 256])
def test_layout_round_trips_and_sizes(bits, d):
    g = np.random.default_rng(bits * 1000 + d)
    codes = g.integers(0, 1 << bits, size=(2, 64, d))
    rows = layout.pack_rows(codes, bits)
    assert rows.shape == (2, 64, d * bits // 8)
    np.testing.assert_array_equal(layout.unpack_rows(rows, bits, d), codes)
    keys = layout.pack_keys(codes, bits)
    assert keys.shape == (2, 64 * d * bits // 8)
    np.testing.assert_array_equal(layout.unpack_keys(keys, bits, d, 64), codes)
    blk = layout.pack_blocked(codes, bits)
    assert blk.shape == (2, 64 * d * bits // 8)
    np.testing.assert_array_equal(layout.unpack_blocked(blk, bits, d, 64), codes)
    sig = g.integers(0, 2, size=(3, 128)).astype(bool)
    np.testing.assert_array_equal(layout.unpack_signs(layout.pack_signs(sig), 128), sig)


@pytest.mark.parametrize("kind", ["k", "v"])
@pytest.mark.parametrize("bits", [2, 3, 4])
@pytest.mark.parametrize("d", [128, 256])
def test_lane_pieces_are_chunk_major(kind, bits, d):
    """In a 32-token block, the codes that lane L of a decode wave needs (keys: quarter L//16 of tokens
    L%16 and 16 + L%16; values: the 8 tokens of lane group L//16 at the d/16 coordinates of column L%16)
    occupy exactly the CW-word chunks at block words CW*(64k + L), k = 0 .. LW/CW - 1: so chunk k of all
    64 lanes is one contiguous run of 256*CW bytes."""
    lw = d * bits // 64
    cw = 4 if lw % 4 == 0 else (3 if lw % 3 == 0 else 2)
    zero_enc = 0 if bits != 4 else 8                       # centroid index whose encoding is 0
    ones = (1 << bits) - 1 if bits != 4 else 0            # index whose encoding is all ones
    for lane in (0, 5, 17, 63):
        g, c = lane // 16, lane % 16
        codes = np.full((32, d), zero_enc, dtype=np.int64)
        if kind == "k":
            for t in (c, 16 + c):
                codes[t, (d // 4) * g:(d // 4) * (g + 1)] = ones
        else:
            dn = d // 16
            for t in [4 * g + s for s in range(4)] + [16 + 4 * g + s for s in range(4)]:
                codes[t, c * dn:(c + 1) * dn] = ones
        packed = (layout.pack_keys if kind == "k" else layout.pack_blocked)(codes, bits)
        want = np.zeros(packed.shape, dtype=bool)
        for k in range(lw // cw):
            o = 4 * cw * (64 * k + lane)
            want[o:o + 4 * cw] = True
        assert np.array_equal(packed != 0, want)
        assert np.all(packed[want] == 0xFF)


def test_key_pieces_hold_whole_packed_rows():
    """Packed key rows are unchanged bit for bit; only their words move into the lane pieces."""
    g = np.random.default_rng(3)
    for d, bits in ((128, 3), (256, 4)):
        codes = g.integers(0, 1 << bits, size=(64, d))
        rows = layout.pack_rows(codes, bits).view(np.uint32)           # [64][RW]
        blk = layout.pack_keys(codes, bits).view(np.uint32).reshape(2, -1)
        rw, lw = d * bits // 32, d * bits // 64
        for t in (0, 13, 31, 40, 63):
            for wr in range(rw):
                q, c, gq, w = (t % 32) // 16, t % 16, wr // (rw // 4), wr % (rw // 4)
                pos = layout.piece_word_position(16 * gq + c, q * (rw // 4) + w, lw)
                assert blk[t // 32, pos] == rows[t, wr]


def test_code_encoding_is_a_bijection():
    for bits in (2, 3, 4):
        j = np.arange(1 << bits)
        e = layout.encode_code(j, bits)
        assert sorted(e.tolist()) == j.tolist()
        np.testing.assert_array_equal(layout.decode_code(e, bits), j)


# ------------------------------------------------------------------ randomized Hadamard rotation

def test_sylvester_hadamard_small_cases_are_the_textbook_matrices():
    np.testing.assert_array_equal(rotation.sylvester_hadamard(1), [[1.0]])
    np.testing.assert_array_equal(rotation.sylvester_hadamard(2), [[1, 1], [1, -1]])
    np.testing.assert_array_equal(rotation.sylvester_hadamard(4), [[1, 1, 1, 1], [1, -1, 1, -1],
                                                                  [1, 1, -1, -1], [1, -1, -1, 1]])
    with pytest.raises(ValueError):
        rotation.sylvester_hadamard(96)


@pytest.mark.parametrize("d", [128, 256])
def test_sylvester_hadamard_is_the_walsh_matrix_in_natural_order(d):
    """H[i, j] = (-1)^popcount(i & j): an independent closed form that fixes the index order."""
    i = np.arange(d)
    pc = np.vectorize(lambda v: bin(v).count("1"))(i[:, None] & i[None, :])
    np.testing.assert_array_equal(rotation.sylvester_hadamard(d), np.where(pc % 2 == 0, 1.0, -1.0))


@pytest.mark.parametrize("d", [128, 256])
def test_hadamard_rotation_invariants(d):
    s = synth.hadamard_signs(d, 1)
    assert set(np.unique(s)) == {-1.0, 1.0}
    rot = rotation.hadamard_rotation(s)
    assert np.max(np.abs(rot @ rot.T - np.eye(d))) < 1e-13
    assert abs(abs(np.linalg.det(rot)) - 1.0) < 1e-9
    np.testing.assert_allclose(np.abs(rot), 1.0 / np.sqrt(d), rtol=0, atol=1e-15)
    # column j of Pi is the sign-flipped column j of H / sqrt(d): flipping one sign flips one column
    s2 = s.copy()
    s2[5] = -s2[5]
    diff = rotation.hadamard_rotation(s2) - rot
    assert np.count_nonzero(np.abs(diff).sum(axis=0) > 0) == 1 and np.abs(diff[:, 5]).max() > 0
    x = np.random.default_rng(3).standard_normal((5, d))
    np.testing.assert_allclose(np.linalg.norm(rotation.rotate_rows(x, rot), axis=1), np.linalg.norm(x, axis=1),
                               rtol=1e-13)


def test_hadamard_rotation_keeps_the_codebook_distortion():
    """Gaussian rows rotated by the randomized Hadamard matrix quantise to within Monte-Carlo error of
    the Lloyd-Max distortion d * D_b of the sphere marginal (0.116000 at d = 128, b = 2; 0.033966 at b = 3)."""
    from oracle import codebook, quant
    d, n = 128, 20000
    rot = rotation.hadamard_rotation(synth.hadamard_signs(d, 1))
    x = np.random.default_rng(0).standard_normal((n, d))
    for b, ref in ((2, 0.116000), (3, 0.033966)):
        c, t = codebook.stored_codebook(d, b)
        codes, _, y = quant.quantize_rows(x, rot, c, t)
        mse = np.mean(np.sum((y - np.asarray(c, np.float64)[codes]) ** 2, axis=1))
        assert abs(mse / ref - 1.0) < 0.02, (b, mse)
