"""Bit layouts of the packed cache (oracle side).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

The pages ask for indices stored in a dense bit stream at unconventional
widths rather than in 8/16-bit boxes (GitHub discussion "TurboQuant support?",
proposal body: a repacked TurboQuant bit-stream format; NVIDIA forum "Why
TurboQuant saves DGX twice", SUMMARY: unconventional bit widths), but print no
layout.  The layouts below are this repository's own specification (format
version 1) and are written out here from their definition.  Parity unpinned by
the pages: the tests pin them with hand-worked byte examples and round trips.

Record layout (keys, QJL signs)
    One record per vector.  Coordinate i's b_i-bit index occupies stream bits
    [o_i, o_i + b_i) with o_i = sum_{k<i} b_k; stream bit p is bit (p mod 8) of
    byte p // 8 (little-endian, LSB first).  Record bytes = sum_i b_i / 8.

Tiled layout (values)
    Tokens are grouped in tiles of 32 consecutive cache positions.  A tile is
    4 token groups (tokens 8g..8g+7) x 16 coordinate groups (coordinates
    8q..8q+7).  Sub-block (g, q) holds 8 coordinates x 8 tokens at width b_q
    (the width of its coordinates) in 8*b_q bytes; inside it the code of
    (coordinate 8q + r, token 8g + s) occupies sub-block stream bits
    [(8r + s) b_q, (8r + s) b_q + b_q).  Sub-blocks are stored g-major:
    offset(g, q) = g * G + sum_{q' < q} 8 b_q', with G = sum_q 8 b_q.
    Tile bytes = 4 G = 32 * record bytes.
"""
from __future__ import annotations

import numpy as np

TILE_TOKENS = 32


def _bits_to_bytes(bits: np.ndarray) -> np.ndarray:
    """[..., 8k] 0/1 array -> [..., k] uint8, bit p -> bit p % 8 of byte p // 8."""
    sh = bits.shape
    b = bits.reshape(sh[:-1] + (sh[-1] // 8, 8)).astype(np.uint8)
    w = (1 << np.arange(8, dtype=np.uint8)).astype(np.uint8)
    return (b * w).sum(axis=-1).astype(np.uint8)


def _bytes_to_bits(by: np.ndarray) -> np.ndarray:
    by = np.asarray(by, dtype=np.uint8)
    bits = (by[..., None] >> np.arange(8, dtype=np.uint8)) & 1
    return bits.reshape(by.shape[:-1] + (by.shape[-1] * 8,))


def _stream_positions(widths: np.ndarray):
    """Per coordinate: the stream bit index of each of its bits (LSB first)."""
    off = np.concatenate(([0], np.cumsum(widths)[:-1]))
    return [off[i] + np.arange(widths[i]) for i in range(len(widths))]


def pack_records(idx: np.ndarray, widths: np.ndarray) -> np.ndarray:
    """idx [n, d] -> records [n, sum(widths)/8] uint8 (record layout)."""
    idx = np.asarray(idx, dtype=np.int64)
    widths = np.asarray(widths, dtype=np.int64)
    total = int(widths.sum())
    if total % 8:
        raise ValueError("record is not a whole number of bytes")
    bits = np.zeros(idx.shape[:-1] + (total,), dtype=np.uint8)
    for i, pos in enumerate(_stream_positions(widths)):
        for k, p in enumerate(pos):
            bits[..., p] = (idx[..., i] >> k) & 1
    return _bits_to_bytes(bits)


def unpack_records(rec: np.ndarray, widths: np.ndarray) -> np.ndarray:
    """records [n, nbytes] -> idx [n, d] int64 (record layout)."""
    widths = np.asarray(widths, dtype=np.int64)
    bits = _bytes_to_bits(rec)
    idx = np.zeros(bits.shape[:-1] + (len(widths),), dtype=np.int64)
    for i, pos in enumerate(_stream_positions(widths)):
        for k, p in enumerate(pos):
            idx[..., i] |= bits[..., p].astype(np.int64) << k
    return idx


def pack_sign_bits(bits: np.ndarray) -> np.ndarray:
    """bool [n, m] -> [n, m/8] uint8: bit j of the sketch at stream bit j."""
    return _bits_to_bytes(np.asarray(bits, dtype=np.uint8))


def unpack_sign_bits(by: np.ndarray) -> np.ndarray:
    return _bytes_to_bits(by).astype(bool)


def tiled_bytes(n_tok: int, widths: np.ndarray) -> int:
    """Bytes of the tiled layout holding ``n_tok`` cache positions (whole tiles)."""
    tiles = -(-n_tok // TILE_TOKENS)
    return tiles * TILE_TOKENS * int(np.sum(widths)) // 8


def _tile_bit_index(widths: np.ndarray):
    """For every (token-in-tile t, coordinate i): the tile stream bit of its code's bit 0.

    Returns an int64 [32, d] array of bit offsets and the per-coordinate width.
    """
    widths = np.asarray(widths, dtype=np.int64)
    d = len(widths)
    if d % 8:
        raise ValueError("d must be a multiple of 8")
    nq = d // 8
    wq = widths.reshape(nq, 8)
    if np.any(wq != wq[:, :1]):
        raise ValueError("every coordinate group of 8 must share one width")
    bq = wq[:, 0]
    sub_bytes = 8 * bq
    group_bytes = int(sub_bytes.sum())
    q_off = np.concatenate(([0], np.cumsum(sub_bytes)[:-1]))
    base = np.zeros((TILE_TOKENS, d), dtype=np.int64)
    for t in range(TILE_TOKENS):
        g, s = divmod(t, 8)
        for i in range(d):
            q, r = divmod(i, 8)
            byte0 = g * group_bytes + q_off[q]
            base[t, i] = 8 * byte0 + (8 * r + s) * bq[q]
    return base, widths


def pack_tiled(idx: np.ndarray, widths: np.ndarray, tok0: int = 0,
               out: np.ndarray | None = None) -> np.ndarray:
    """Write codes of tokens tok0 .. tok0+n-1 (idx [n, d]) into a tiled buffer.

    ``out`` (uint8, whole tiles) is updated in place when given, so positions
    outside the written range keep their previous codes; otherwise a zeroed
    buffer just large enough is created.
    """
    idx = np.asarray(idx, dtype=np.int64)
    n = idx.shape[0]
    base, widths = _tile_bit_index(widths)
    need = tiled_bytes(tok0 + n, widths)
    if out is None:
        out = np.zeros(need, dtype=np.uint8)
    if out.size < need:
        raise ValueError("tiled buffer too small")
    bits = _bytes_to_bits(out).copy()
    tile_bits = TILE_TOKENS * int(widths.sum())
    for j in range(n):
        p = tok0 + j
        tile, t = divmod(p, TILE_TOKENS)
        for i in range(len(widths)):
            for k in range(widths[i]):
                bits[tile * tile_bits + base[t, i] + k] = (idx[j, i] >> k) & 1
    out[:] = _bits_to_bytes(bits)
    return out


def unpack_tiled(buf: np.ndarray, widths: np.ndarray, n_tok: int, tok0: int = 0) -> np.ndarray:
    """Read codes of tokens tok0 .. tok0+n_tok-1 from a tiled buffer -> [n_tok, d]."""
    base, widths = _tile_bit_index(widths)
    bits = _bytes_to_bits(np.asarray(buf, dtype=np.uint8))
    tile_bits = TILE_TOKENS * int(widths.sum())
    pos = tok0 + np.arange(n_tok)
    tile, t = np.divmod(pos, TILE_TOKENS)
    start = tile[:, None] * tile_bits + base[t, :]          # [n_tok, d]
    idx = np.zeros((n_tok, len(widths)), dtype=np.int64)
    for k in range(int(widths.max())):
        has = widths > k
        val = bits[np.where(has[None, :], start + k, 0)].astype(np.int64)
        idx |= np.where(has[None, :], val, 0) << k
    return idx
