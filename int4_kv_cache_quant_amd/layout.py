"""Index maps between the cache's code layouts and the plain token-major
layout (pure permutations of nibbles; no arithmetic).

Plain layout: codes[..., token, D/2], byte j = element 2j (low nibble) and
2j+1 (high nibble).  K row layout (include/otq.h): 32-bit word r * NG + g of
a row holds channels 32 g + 8 r + 0..7.  V tile layout: per tile of 32 tokens,
16*D bytes; tile-relative token u has quarter r = (u % 16) // 4 and slot
j = 4 * (u // 16) + u % 4; channel c = 16 * (4a + b) + n owns word
((a*4 + r)*16 + n)*4 + b; slot j is nibble j % 2 of byte j // 2 of that word.
"""
import functools

import numpy as np


@functools.lru_cache(maxsize=None)
def _tile_maps(D):
    o = np.arange(16 * D)
    word, byte = o // 4, o % 4
    b = word % 4
    n = (word // 4) % 16
    r = (word // 64) % 4
    a = word // 256
    c = 16 * (4 * a + b) + n
    # nibble x of tile byte o holds slot j = 2 * byte + x
    us, cs = [], []
    for x in (0, 1):
        j = 2 * byte + x
        us.append(16 * (j // 4) + 4 * r + (j % 4))
        cs.append(c)
    return np.stack(us, -1), np.stack(cs, -1)   # [16D, 2] token, channel


def _nibbles(packed):
    p = np.asarray(packed, np.uint8)
    return np.stack([p & 0xF, p >> 4], -1)


def v_tiled_to_plain(tiled, D):
    """[..., C/32, 16*D] tile layout -> [..., C, D/2] plain layout."""
    tiled = np.asarray(tiled, np.uint8)
    lead, ntile = tiled.shape[:-2], tiled.shape[-2]
    u, c = _tile_maps(D)
    nib = _nibbles(tiled)                                    # [..., ntile, 16D, 2]
    plain = np.zeros(lead + (ntile, 32, D), np.uint8)
    plain[..., u, c] = nib
    plain = plain.reshape(lead + (ntile * 32, D // 2, 2))
    return (plain[..., 0] | (plain[..., 1] << 4)).astype(np.uint8)


def v_plain_to_tiled(plain, D):
    """[..., C, D/2] plain layout -> [..., C/32, 16*D] tile layout."""
    plain = np.asarray(plain, np.uint8)
    lead, C = plain.shape[:-2], plain.shape[-2]
    nib = _nibbles(plain).reshape(lead + (C // 32, 32, D))
    u, c = _tile_maps(D)
    t = nib[..., u, c]                                       # [..., C/32, 16D, 2]
    return (t[..., 0] | (t[..., 1] << 4)).astype(np.uint8)


@functools.lru_cache(maxsize=None)
def _k_row_map(D):
    """plain byte index held by each K-row byte (same nibble order)."""
    NG = D // 32
    idx = np.zeros(D // 2, np.int64)
    for c in range(0, D, 2):
        g, r, k = c // 32, (c // 8) % 4, c % 8
        idx[(r * NG + g) * 4 + k // 2] = c // 2
    return idx


def k_rows_to_plain(rows, D):
    """[..., T, D/2] K row layout -> [..., T, D/2] plain layout."""
    rows = np.asarray(rows, np.uint8)
    out = np.empty_like(rows)
    out[..., _k_row_map(D)] = rows
    return out


def k_plain_to_rows(plain, D):
    """[..., T, D/2] plain layout -> [..., T, D/2] K row layout."""
    return np.asarray(plain, np.uint8)[..., _k_row_map(D)]


# ---------------------------------------------------------------- b-bit V tiles
# Plain b-bit rows: element c of a token's row at bits [b c, b c + b) of the
# row's little-endian bit stream.  V tile layout of 2- and 3-bit caches
# (include/otq.h): per tile of 32 tokens, 32 D b / 8 bytes; tile-relative
# token u has h = u // 16, r = (u % 16) // 4, m = u % 4; channel c has
# cb = c // 16, n = c % 16; lane l = 16 r + n.
#   2 bits: word l (D/32) + cb // 2, field at bit 16 h + 8 (cb % 2) + 2 m.
#   3 bits: words l (3D/64) + 3 (cb // 4) + w; for w = cb % 4 < 3 the field at
#           bit 16 h + 3 m of word w; for cb % 4 = 3, bit i of the field is
#           chunk bit p = 3 m + i, at bit 16 h + 12 + p % 4 of word p // 4.
# Tile bit index = 32 word + bit (little-endian bytes).

@functools.lru_cache(maxsize=None)
def _vbits_map(D, bits):
    """src[t]: the plain bit (u * D * bits + c * bits + i) that tile bit t holds."""
    u = np.arange(32)[:, None, None]
    c = np.arange(D)[None, :, None]
    i = np.arange(bits)[None, None, :]
    h, r, m = u // 16, (u % 16) // 4, u % 4
    cb, n = c // 16, c % 16
    lane = 16 * r + n
    if bits == 2:
        word = lane * (D // 32) + cb // 2
        bit = 16 * h + 8 * (cb % 2) + 2 * m + i
    elif bits == 3:
        wpl = 3 * D // 64
        qd, w = cb // 4, cb % 4
        p = 3 * m + i
        word = np.where(w < 3, lane * wpl + 3 * qd + w, lane * wpl + 3 * qd + p // 4)
        bit = np.where(w < 3, 16 * h + 3 * m + i, 16 * h + 12 + p % 4)
    else:
        raise ValueError("2- or 3-bit codes")
    word, bit = np.broadcast_arrays(word, bit)
    tbit = (32 * word + bit).reshape(-1)
    plain = (u * D * bits + c * bits + i)
    plain = np.broadcast_to(plain, word.shape).reshape(-1)
    src = np.full(32 * D * bits, -1, np.int64)
    src[tbit] = plain
    return src


def v_bits_plain_to_tiled(plain, D, bits):
    """[..., C, D*bits/8] plain rows -> [..., C/32, 32*D*bits/8] tile layout."""
    plain = np.asarray(plain, np.uint8)
    lead, C = plain.shape[:-2], plain.shape[-2]
    pb = np.unpackbits(plain.reshape(lead + (C // 32, 32 * D * bits // 8)), axis=-1, bitorder="little")
    tb = pb[..., _vbits_map(D, bits)]
    return np.packbits(tb, axis=-1, bitorder="little")


def v_bits_tiled_to_plain(tiled, D, bits):
    """[..., C/32, 32*D*bits/8] tile layout -> [..., C, D*bits/8] plain rows."""
    tiled = np.asarray(tiled, np.uint8)
    lead, ntile = tiled.shape[:-2], tiled.shape[-2]
    tb = np.unpackbits(tiled, axis=-1, bitorder="little")
    pb = np.empty_like(tb)
    pb[..., _vbits_map(D, bits)] = tb
    return np.packbits(pb, axis=-1, bitorder="little").reshape(lead + (ntile * 32, D * bits // 8))
