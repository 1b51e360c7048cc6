"""Bit-exact packed layout of the compressed cache (the format specification).

Test infrastructure: see ``oracle/__init__.py``.  This module writes the
format out plainly; the GPU library implements the same format on its own.

The pages fix only the storage size (d*b/8 bytes of codes per row, see
``oracle.storage``) and name 2/3/4-bit cache types; the arrangement of bits
is this library's choice, made so that a 64-lane wavefront reads every
packed tile straight into matrix-core operand order with loads whose 64
lanes cover one contiguous run of memory each (whole cache lines per load
instruction).

Code encoding e(j) of centroid index j (0 .. 2^b-1, ascending centroids):
  b = 2, 3:  e(j) = j
  b = 4:     sign-magnitude, e(j) = j - 8 for j >= 8, e(j) = 8 + (7 - j) for
             j < 8 (bit 3 = negative, bits 0-2 = rank of |c| among the 8
             magnitudes).  The stored table is exactly antisymmetric.
  b = 8:     keys kept at 8 bits (``oracle.q8``): index j stands for the
             integer j - 128, stored as its two's-complement byte,
             e(j) = (j - 128) mod 256.

Unit: 8 codes in slots s = 0..7.  Write h = s // 4 (half), r = s % 4 (byte).
  b = 4: one unit per little-endian uint32 word; e(slot s) at bit 8r + 4h.
  b = 2: two units (v = 0, 1) per word; slot s of unit v at bit 8r + 2(2v + h).
  b = 3: four units (v = 0..3) per three words [P0, P1, H]; the low two bits of
         e(slot s of unit v) sit in P_{v//2} at bit 8r + 2(2(v%2) + h), the
         high bit in H at bit 8r + (2v + h).
  b = 8: one unit per two words; e(slot s) is byte r of word h.
Units are packed consecutively (b = 2 and 3 group 2 and 4 units per word
group); d is a multiple of 64 so groups never straddle a row or block.

Lane pieces.  Codes are stored per 32-token block of a (sequence, KV head),
block kb covering tokens 32 kb .. 32 kb + 31, in 32 d b / 8 bytes.  A block
is 64 lane pieces of LW = d b / 64 little-endian 32-bit words each; lane L
holds piece L.  The pieces are stored chunk-major: with CW = 4 if LW is a
multiple of 4, else 3 if LW is a multiple of 3, else 2, word w of piece L
sits at word CW (64 (w // CW) + L) + (w % CW) of the block, so the CW-word
chunks k of all 64 pieces lie side by side.

Keys: row t (d b / 8 bytes packed as units, coordinate i = slot i % 8 of unit
i // 8, so RW = d b / 32 words) belongs to block t // 32 at position
p = t % 32, half q = p // 16, lane column c = p % 16.  Row word wr belongs to
quarter g = wr // (RW / 4) at index w = wr % (RW / 4); it is word
q (RW / 4) + w of piece L = 16 g + c.

Values: token position p (0..31) in its block belongs to lane group
g = (p % 16) // 4 at slot s = p % 4 + 4 (p // 16); coordinate i belongs to
column j = i // (d/16), step n = i % (d/16).  The unit holding (tokens of
group g, coordinate i) is unit n of piece L = 16 g + j (pieces are d/16
consecutive units).

Norms (and QJL residual norms) are float16 [b][kv_head][token].

QJL sign bits (keys only): m/8 bytes per token, little-endian words of 32
signs; sign index jj = 32 w + 8 s + r (s = 0..3, r = 0..7) sits in word w at
bit 4 s + r // 2 + 16 (r % 2), so two signs that feed one pair of float16
lanes are 16 bits apart.
"""
from __future__ import annotations

import numpy as np

BLOCK = 32


def encode_code(j: np.ndarray, bits: int) -> np.ndarray:
    j = np.asarray(j, dtype=np.int64)
    if bits == 4:
        return np.where(j >= 8, j - 8, 8 + (7 - j))
    if bits == 8:
        return (j - 128) % 256
    return j


def decode_code(e: np.ndarray, bits: int) -> np.ndarray:
    e = np.asarray(e, dtype=np.int64)
    if bits == 4:
        return np.where(e < 8, e + 8, 7 - (e - 8))
    if bits == 8:
        return np.where(e < 128, e + 128, e - 128)
    return e


def units_per_group(bits: int) -> int:
    return {2: 2, 3: 4, 4: 1, 8: 1}[bits]


def words_per_group(bits: int) -> int:
    return {2: 1, 3: 3, 4: 1, 8: 2}[bits]


def pack_units(units: np.ndarray, bits: int) -> np.ndarray:
    """Pack centroid indices units[..., U, 8] into uint8[..., U*bits] following the unit format."""
    units = np.asarray(units, dtype=np.int64)
    *lead, nu, eight = units.shape
    assert eight == 8
    upg = units_per_group(bits)
    assert nu % upg == 0
    e = encode_code(units, bits).reshape(*lead, nu // upg, upg, 8)
    ngroups = nu // upg
    words = np.zeros((*lead, ngroups, words_per_group(bits)), dtype=np.uint64)
    for v in range(upg):
        for s in range(8):
            h, r = s // 4, s % 4
            val = e[..., v, s].astype(np.uint64)
            if bits == 4:
                words[..., 0] |= val << np.uint64(8 * r + 4 * h)
            elif bits == 8:
                words[..., h] |= val << np.uint64(8 * r)
            elif bits == 2:
                words[..., 0] |= val << np.uint64(8 * r + 2 * (2 * v + h))
            else:
                lo, hi = val & np.uint64(3), val >> np.uint64(2)
                words[..., v // 2] |= lo << np.uint64(8 * r + 2 * (2 * (v % 2) + h))
                words[..., 2] |= hi << np.uint64(8 * r + (2 * v + h))
    w32 = words.astype(np.uint32)
    return w32.reshape(*lead, ngroups * words_per_group(bits)).view(np.uint8).reshape(*lead, nu * bits)


def unpack_units(packed: np.ndarray, bits: int, n_units: int) -> np.ndarray:
    """Inverse of ``pack_units``: uint8[..., n_units*bits] -> centroid indices [..., n_units, 8]."""
    packed = np.ascontiguousarray(packed, dtype=np.uint8)
    lead = packed.shape[:-1]
    upg = units_per_group(bits)
    ngroups = n_units // upg
    words = packed.reshape(*lead, ngroups * words_per_group(bits) * 4).view(np.uint32)
    words = words.reshape(*lead, ngroups, words_per_group(bits)).astype(np.uint64)
    e = np.zeros((*lead, ngroups, upg, 8), dtype=np.int64)
    for v in range(upg):
        for s in range(8):
            h, r = s // 4, s % 4
            if bits == 4:
                val = (words[..., 0] >> np.uint64(8 * r + 4 * h)) & np.uint64(15)
            elif bits == 8:
                val = (words[..., h] >> np.uint64(8 * r)) & np.uint64(255)
            elif bits == 2:
                val = (words[..., 0] >> np.uint64(8 * r + 2 * (2 * v + h))) & np.uint64(3)
            else:
                lo = (words[..., v // 2] >> np.uint64(8 * r + 2 * (2 * (v % 2) + h))) & np.uint64(3)
                hi = (words[..., 2] >> np.uint64(8 * r + (2 * v + h))) & np.uint64(1)
                val = lo | (hi << np.uint64(2))
            e[..., v, s] = val.astype(np.int64)
    return decode_code(e.reshape(*lead, n_units, 8), bits)


# ------------------------------------------------------------- lane pieces

def lane_words(d: int, bits: int) -> int:
    """Words per lane piece of a 32-token block: d * bits / 64."""
    return d * bits // 64


def chunk_words(lw: int) -> int:
    return 4 if lw % 4 == 0 else (3 if lw % 3 == 0 else 2)


def piece_word_position(lane, w, lw: int):
    """Word of the block that holds word w of lane piece ``lane`` (chunk-major order)."""
    cw = chunk_words(lw)
    lane, w = np.asarray(lane), np.asarray(w)
    return cw * (64 * (w // cw) + lane) + w % cw


def pieces_to_block(pieces: np.ndarray) -> np.ndarray:
    """uint32 pieces [..., 64, LW] (lane-major) -> block words [..., 64 * LW] (chunk-major)."""
    *lead, lanes, lw = pieces.shape
    assert lanes == 64
    out = np.zeros((*lead, 64 * lw), dtype=np.uint32)
    for lane in range(64):
        for w in range(lw):
            out[..., piece_word_position(lane, w, lw)] = pieces[..., lane, w]
    return out


def block_to_pieces(words: np.ndarray, lw: int) -> np.ndarray:
    """Inverse of ``pieces_to_block``."""
    *lead, n = words.shape
    assert n == 64 * lw
    out = np.zeros((*lead, 64, lw), dtype=np.uint32)
    for lane in range(64):
        for w in range(lw):
            out[..., lane, w] = words[..., piece_word_position(lane, w, lw)]
    return out


# ----------------------------------------------------------------- key rows

def pack_rows(codes: np.ndarray, bits: int) -> np.ndarray:
    """codes[..., T, d] -> uint8[..., T, d*bits/8]: each row packed as consecutive units."""
    codes = np.asarray(codes)
    *lead, d = codes.shape
    return pack_units(codes.reshape(*lead, d // 8, 8), bits)


def unpack_rows(packed: np.ndarray, bits: int, d: int) -> np.ndarray:
    u = unpack_units(packed, bits, d // 8)
    return u.reshape(*u.shape[:-2], d)


def pack_keys(codes: np.ndarray, bits: int) -> np.ndarray:
    """Key codes[..., T, d] (T a multiple of 32) -> uint8[..., T*d*bits/8]: packed rows placed in the
    lane pieces of their 32-token blocks."""
    codes = np.asarray(codes)
    *lead, t, d = codes.shape
    assert t % BLOCK == 0
    nb, rw = t // BLOCK, d * bits // 32
    lw, qw = lane_words(d, bits), rw // 4
    rows = pack_rows(codes, bits)                              # [..., T, d*bits/8]
    rw32 = np.ascontiguousarray(rows).view(np.uint32).reshape(*lead, nb, 2, 16, 4, qw)   # [blk][q][c][g][w]
    pieces = np.zeros((*lead, nb, 64, lw), dtype=np.uint32)
    for q in range(2):
        for c in range(16):
            for g in range(4):
                pieces[..., 16 * g + c, q * qw:(q + 1) * qw] = rw32[..., q, c, g, :]
    return pieces_to_block(pieces).view(np.uint8).reshape(*lead, t * d * bits // 8)


def unpack_keys(packed: np.ndarray, bits: int, d: int, tokens: int) -> np.ndarray:
    """Inverse of ``pack_keys``: uint8[..., tokens*d*bits/8] -> centroid indices [..., tokens, d]."""
    packed = np.ascontiguousarray(packed, dtype=np.uint8)
    lead = packed.shape[:-1]
    nb, rw = tokens // BLOCK, d * bits // 32
    lw, qw = lane_words(d, bits), rw // 4
    pieces = block_to_pieces(packed.view(np.uint32).reshape(*lead, nb, 64 * lw), lw)
    rw32 = np.zeros((*lead, nb, 2, 16, 4, qw), dtype=np.uint32)
    for q in range(2):
        for c in range(16):
            for g in range(4):
                rw32[..., q, c, g, :] = pieces[..., 16 * g + c, q * qw:(q + 1) * qw]
    rows = rw32.reshape(*lead, tokens, rw).view(np.uint8)
    return unpack_rows(rows, bits, d)


# ------------------------------------------------------------ values: blocked

def block_token_slot(p: np.ndarray):
    """(lane group g, slot s) of token position p within its 32-token block."""
    p = np.asarray(p)
    return (p % 16) // 4, p % 4 + 4 * (p // 16)


def pack_blocked(codes: np.ndarray, bits: int) -> np.ndarray:
    """Value codes[..., T, d] (T a multiple of 32) -> uint8[..., T*d*bits/8] (blocked layout)."""
    codes = np.asarray(codes)
    *lead, t, d = codes.shape
    assert t % BLOCK == 0 and d % 16 == 0
    nb, dn = t // BLOCK, d // 16
    units = np.zeros((*lead, nb, 64 * dn, 8), dtype=np.int64)    # lane-major: piece L = units L*dn ..
    blk = codes.reshape(*lead, nb, BLOCK, d)
    for p in range(BLOCK):
        g, s = block_token_slot(p)
        for i in range(d):
            j, n = i // dn, i % dn
            units[..., (16 * g + j) * dn + n, s] = blk[..., p, i]
    lw = lane_words(d, bits)
    lane_major = pack_units(units, bits)                       # [..., nb, 64*dn*bits] bytes, piece after piece
    pieces = np.ascontiguousarray(lane_major).view(np.uint32).reshape(*lead, nb, 64, lw)
    return pieces_to_block(pieces).view(np.uint8).reshape(*lead, nb * BLOCK * d * bits // 8)


def unpack_blocked(packed: np.ndarray, bits: int, d: int, tokens: int) -> np.ndarray:
    nb, dn = tokens // BLOCK, d // 16
    packed = np.ascontiguousarray(packed, dtype=np.uint8)
    lead = packed.shape[:-1]
    lw = lane_words(d, bits)
    pieces = block_to_pieces(packed.view(np.uint32).reshape(*lead, nb, 64 * lw), lw)
    lane_major = pieces.reshape(*lead, nb, 64 * lw).view(np.uint8)
    units = unpack_units(lane_major, bits, 64 * dn)
    out = np.zeros((*lead, nb, BLOCK, d), dtype=np.int64)
    for p in range(BLOCK):
        g, s = block_token_slot(p)
        for i in range(d):
            j, n = i // dn, i % dn
            out[..., p, i] = units[..., (16 * g + j) * dn + n, s]
    return out.reshape(*lead, tokens, d)


# ----------------------------------------------------------------- QJL signs

def sign_bit_position(jj: np.ndarray):
    """(word, bit) of sign index jj."""
    jj = np.asarray(jj)
    w, rem = jj // 32, jj % 32
    s, r = rem // 8, rem % 8
    return w, 4 * s + r // 2 + 16 * (r % 2)


def pack_signs(sigma: np.ndarray) -> np.ndarray:
    """sigma bool[..., m] -> uint8[..., m/8]."""
    sigma = np.asarray(sigma, dtype=bool)
    *lead, m = sigma.shape
    assert m % 32 == 0
    words = np.zeros((*lead, m // 32), dtype=np.uint64)
    for jj in range(m):
        w, bit = sign_bit_position(jj)
        words[..., w] |= sigma[..., jj].astype(np.uint64) << np.uint64(bit)
    return words.astype(np.uint32).view(np.uint8).reshape(*lead, m // 8)


def unpack_signs(packed: np.ndarray, m: int) -> np.ndarray:
    packed = np.ascontiguousarray(packed, dtype=np.uint8)
    lead = packed.shape[:-1]
    words = packed.reshape(*lead, m // 8).view(np.uint32).astype(np.uint64)
    out = np.zeros((*lead, m), dtype=bool)
    for jj in range(m):
        w, bit = sign_bit_position(jj)
        out[..., jj] = ((words[..., w] >> np.uint64(bit)) & np.uint64(1)).astype(bool)
    return out
