"""Test-side writer and reader of the quantized-activation record layout (numpy).

Written from the layout that include/dq.h documents for dq_quantize_act's
output: records of 5120 bytes, one per (super-block b, 16-row block mb), at
(b * MB + mb) * 5120 with MB = ceil(M / 16); inside a record the codes of row
r, 16-byte unit u at r * 256 + 16 * (u ^ r); the 32-value code sums of row r,
group j at 4096 + r * 32 + 4 * j as two binary16 values (s & 63, s - (s & 63));
d_x of row r at 4608 + 4 * r; zeros from 4672 on.  Rows past M are zero.
"""
from __future__ import annotations

import numpy as np

RECORD = 5120
SUMS, DX, PAD = 4096, 4608, 4672


def act_bytes(M: int, K: int) -> int:
    return -(-M // 16) * (K // 256) * RECORD


def pack(q: np.ndarray, d: np.ndarray, bsum: np.ndarray) -> np.ndarray:
    """(q int8 [M, K], d f32 [M, K/256], bsum int32 [M, K/32]) -> uint8 buffer."""
    M, K = q.shape
    nb, nmb = K // 256, -(-M // 16)
    out = np.zeros(act_bytes(M, K), np.uint8)
    recs = out.reshape(nb, nmb, RECORD)
    for m in range(M):
        mb, r = divmod(m, 16)
        for b in range(nb):
            rec = recs[b, mb]
            codes = q[m, 256 * b:256 * (b + 1)].view(np.uint8).reshape(16, 16)
            for u in range(16):
                pos = r * 256 + 16 * (u ^ r)
                rec[pos:pos + 16] = codes[u]
            for j in range(8):
                s = int(bsum[m, 8 * b + j])
                lo = s & 63
                pair = np.array([lo, s - lo], np.float16)
                assert int(pair[0]) + int(pair[1]) == s
                rec[SUMS + 32 * r + 4 * j:SUMS + 32 * r + 4 * j + 4] = pair.view(np.uint8)
            rec[DX + 4 * r:DX + 4 * r + 4] = np.array([d[m, b]], np.float32).view(np.uint8)
    return out


def unpack(buf: np.ndarray, M: int, K: int):
    """uint8 buffer -> (q, d, bsum, padding_ok): padding_ok checks the zero rows and tails."""
    buf = np.asarray(buf, np.uint8)
    nb, nmb = K // 256, -(-M // 16)
    assert buf.size >= act_bytes(M, K)
    recs = buf[:act_bytes(M, K)].reshape(nb, nmb, RECORD)
    q = np.zeros((M, K), np.int8)
    d = np.zeros((M, nb), np.float32)
    bsum = np.zeros((M, K // 32), np.int32)
    padding_ok = not recs[:, :, PAD:].any()
    for mb in range(nmb):
        for r in range(16):
            m = 16 * mb + r
            for b in range(nb):
                rec = recs[b, mb]
                row = np.concatenate([rec[r * 256 + 16 * (u ^ r):r * 256 + 16 * (u ^ r) + 16]
                                      for u in range(16)])
                pairs = rec[SUMS + 32 * r:SUMS + 32 * r + 32].view(np.float16).astype(np.int64)
                sums = pairs[0::2] + pairs[1::2]
                dx = rec[DX + 4 * r:DX + 4 * r + 4].view(np.float32)[0]
                if m >= M:
                    padding_ok &= not row.any() and not sums.any() and dx == 0
                    continue
                q[m, 256 * b:256 * (b + 1)] = row.view(np.int8)
                bsum[m, 8 * b:8 * b + 8] = sums
                d[m, b] = dx
                padding_ok &= bool(np.all(pairs[0::2] == (sums & 63)))
    return q, d, bsum, padding_ok
