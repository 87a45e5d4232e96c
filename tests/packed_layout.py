"""Test-side reader of the repacked tile layout (numpy, CPU).

Written from the layout description in the library's private header: tiles of
16 weight rows x one super-block, n-tile-major; per-lane 16-byte records for
the 16x16x64 int8 matrix instruction (lane l: row l % 16, quarter kq = l // 16,
codes of chunk c at k = 64kq + 16c + p).  Used to check that the repack moves every code,
scale and header bit to where the layout says, and nothing else.
"""
from __future__ import annotations

import numpy as np

Q4_K, Q6_K = 12, 14
TILE = {Q4_K: 2304, Q6_K: 3360}
ROWS = 16


def _nibble_records(rec: np.ndarray) -> np.ndarray:
    """rec [2 records][64 lanes][16 B] -> 4-bit parts q[16 rows][256 k]."""
    out = np.zeros((16, 256), np.int64)
    for i in range(2):
        for lane in range(64):
            r, kq = lane % 16, lane // 16
            for t in range(4):
                c, h = 2 * i + t // 2, t % 2
                for e in range(4):
                    byte = int(rec[i, lane, 4 * t + e])
                    k = 64 * kq + 16 * c + 8 * h + e
                    out[r, k] = byte & 15
                    out[r, k + 4] = byte >> 4
    return out


def read_tile(type_: int, tile: np.ndarray):
    """Decode one tile.  Q4_K -> (heads [16,16] bytes, q [16,256]);
    Q6_K -> (d_bits [16] uint16, sc [16,16] int8, q [16,256])."""
    tile = np.asarray(tile, np.uint8)
    if type_ == Q4_K:
        heads = tile[:256].reshape(16, 16)
        q = _nibble_records(tile[256:2304].reshape(2, 64, 16))
        return heads, q
    low = _nibble_records(tile[:2048].reshape(2, 64, 16))
    qh = tile[2048:3072].reshape(64, 16)
    high = np.zeros((16, 256), np.int64)
    for lane in range(64):
        r, kq = lane % 16, lane // 16
        for c in range(4):
            for e in range(4):
                byte = int(qh[lane, 4 * c + e])
                for s in range(4):
                    p = 4 * s + e
                    high[r, 64 * kq + 16 * c + p] = (byte >> (2 * s)) & 3
    scp = tile[3072:3328].reshape(4, 16, 4).view(np.int8)
    sc = np.zeros((16, 16), np.int64)
    for kq in range(4):
        for c in range(4):
            sc[:, 4 * kq + c] = scp[kq, :, c]
    d_bits = tile[3328:3360].view(np.uint16)
    return d_bits, sc, low | (high << 4)
