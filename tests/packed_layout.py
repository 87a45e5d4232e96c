"""Test-side reader of the repacked tile layout (numpy, CPU).

Written from the layout description in the library's private header: tiles of
32 weight rows x one super-block, n-tile-major; per-lane 16-byte records for
the 32x32x32 int8 matrix instruction (lane l: row l % 32, half g = l // 32,
codes of chunk c at k = 128g + 16c + p).  Used to check that the repack moves every code,
scale and header bit to where the layout says, and nothing else.
"""
from __future__ import annotations

import numpy as np

Q4_K, Q6_K = 12, 14
TILE = {Q4_K: 4608, Q6_K: 6720}


def _nibble_records(rec: np.ndarray) -> np.ndarray:
    """rec [4 records][64 lanes][16 B] -> 4-bit parts q[32 rows][256 k]."""
    out = np.zeros((32, 256), np.int64)
    for i in range(4):
        for lane in range(64):
            r, g = lane % 32, lane // 32
            for t in range(4):
                c, h = 2 * i + t // 2, t % 2
                for e in range(4):
                    byte = int(rec[i, lane, 4 * t + e])
                    k = 128 * g + 16 * c + 8 * h + e
                    out[r, k] = byte & 15
                    out[r, k + 4] = byte >> 4
    return out


def read_tile(type_: int, tile: np.ndarray):
    """Decode one tile.  Q4_K -> (heads [32,16] bytes, q [32,256]);
    Q6_K -> (d_bits [32] uint16, sc [32,16] int8, q [32,256])."""
    tile = np.asarray(tile, np.uint8)
    if type_ == Q4_K:
        heads = tile[:512].reshape(32, 16)
        q = _nibble_records(tile[512:4608].reshape(4, 64, 16))
        return heads, q
    low = _nibble_records(tile[:4096].reshape(4, 64, 16))
    qh = tile[4096:6144].reshape(2, 64, 16)
    high = np.zeros((32, 256), np.int64)
    for i in range(2):
        for lane in range(64):
            r, g = lane % 32, lane // 32
            for t in range(4):
                c = 4 * i + t
                for e in range(4):
                    byte = int(qh[i, lane, 4 * t + e])
                    for s in range(4):
                        p = 4 * s + e
                        high[r, 128 * g + 16 * c + p] = (byte >> (2 * s)) & 3
    scp = tile[6144:6656].reshape(2, 32, 8).view(np.int8)
    sc = np.zeros((32, 16), np.int64)
    for g in range(2):
        for c in range(8):
            sc[:, 8 * g + c] = scp[g, :, c]
    d_bits = tile[6656:6720].view(np.uint16)
    return d_bits, sc, low | (high << 4)
