"""Field-level K-quant blocks for the oracle pins (test-side only).

The oracle decodes bytes -> fields by walking the bytes.  This module goes the
other way, fields -> bytes, by asking for every weight and every scale which
byte and which bits hold it (the GGUF/ggml Q4_K and Q6_K block definitions;
the pages name the types but not their bytes).  Being the inverse map, written
per weight instead of per byte, a misread position in either one shows up as a
round-trip mismatch.  Brute-force references in the tests use the fields
directly, never the oracle's decoder.
"""
from __future__ import annotations

import numpy as np


def q4k_position(i: int):
    """Byte index within qs and bit shift of the 4-bit code of weight i."""
    c, r = divmod(i, 64)
    return 32 * c + (r % 32), (4 if r >= 32 else 0)


def q4k_scale_bits(j: int):
    """[(byte, shift, width, value_shift)] pieces of sc_j and of mn_j in scales[12]."""
    if j < 4:
        sc = [(j, 0, 6, 0)]
        mn = [(j + 4, 0, 6, 0)]
    else:
        sc = [(j + 4, 0, 4, 0), (j - 4, 6, 2, 4)]
        mn = [(j + 4, 4, 4, 0), (j, 6, 2, 4)]
    return sc, mn


def enc_q4k(d: float, dmin: float, sc, mn, q) -> np.ndarray:
    """Fields -> one 144-byte Q4_K block.  d, dmin as fp16; sc, mn in [0,63]; q in [0,15]."""
    blk = np.zeros(144, np.uint8)
    blk[0:2] = np.array([d], np.float16).view(np.uint8)
    blk[2:4] = np.array([dmin], np.float16).view(np.uint8)
    s = np.zeros(12, np.int64)
    for j in range(8):
        sp, mp = q4k_scale_bits(j)
        for (byte, shift, width, vshift) in sp:
            s[byte] |= ((int(sc[j]) >> vshift) & ((1 << width) - 1)) << shift
        for (byte, shift, width, vshift) in mp:
            s[byte] |= ((int(mn[j]) >> vshift) & ((1 << width) - 1)) << shift
    blk[4:16] = s.astype(np.uint8)
    qs = np.zeros(128, np.int64)
    for i in range(256):
        byte, shift = q4k_position(i)
        qs[byte] |= (int(q[i]) & 15) << shift
    blk[16:144] = qs.astype(np.uint8)
    return blk


def q6k_position(i: int):
    """(ql byte, ql shift, qh byte, qh shift) of the 6-bit code of weight i."""
    h, r = divmod(i, 128)
    quarter, l = divmod(r, 32)
    ql_byte = 64 * h + l + (32 if quarter in (1, 3) else 0)
    ql_shift = 4 if quarter >= 2 else 0
    return ql_byte, ql_shift, 32 * h + l, 2 * quarter


def enc_q6k(d: float, sc, q) -> np.ndarray:
    """Fields -> one 210-byte Q6_K block.  d as fp16; sc int8 [16]; q in [0,63] [256]."""
    blk = np.zeros(210, np.uint8)
    ql = np.zeros(128, np.int64)
    qh = np.zeros(64, np.int64)
    for i in range(256):
        qb, qsft, hb, hsft = q6k_position(i)
        ql[qb] |= (int(q[i]) & 15) << qsft
        qh[hb] |= ((int(q[i]) >> 4) & 3) << hsft
    blk[0:128] = ql.astype(np.uint8)
    blk[128:192] = qh.astype(np.uint8)
    blk[192:208] = np.asarray(sc, np.int8).view(np.uint8)
    blk[208:210] = np.array([d], np.float16).view(np.uint8)
    return blk


def random_q4k_fields(rng, N, nb):
    d = (np.abs(rng.standard_normal((N, nb))) * 2e-3).astype(np.float16)
    dmin = (np.abs(rng.standard_normal((N, nb))) * 2e-3).astype(np.float16)
    sc = rng.integers(0, 64, (N, nb, 8))
    mn = rng.integers(0, 64, (N, nb, 8))
    q = rng.integers(0, 16, (N, nb, 256))
    return dict(d=d, dmin=dmin, sc=sc, mn=mn, q=q)


def random_q6k_fields(rng, N, nb, sc_lo=-128, sc_hi=127):
    d = (np.abs(rng.standard_normal((N, nb))) * 2e-3).astype(np.float16)
    sc = rng.integers(sc_lo, sc_hi + 1, (N, nb, 16))
    q = rng.integers(0, 64, (N, nb, 256))
    return dict(d=d, sc=sc, q=q)


def encode_q4k_matrix(f) -> np.ndarray:
    N, nb = f["d"].shape
    out = np.zeros((N, nb, 144), np.uint8)
    for n in range(N):
        for b in range(nb):
            out[n, b] = enc_q4k(f["d"][n, b], f["dmin"][n, b], f["sc"][n, b], f["mn"][n, b],
                                f["q"][n, b])
    return out


def encode_q6k_matrix(f) -> np.ndarray:
    N, nb = f["d"].shape
    out = np.zeros((N, nb, 210), np.uint8)
    for n in range(N):
        for b in range(nb):
            out[n, b] = enc_q6k(f["d"][n, b], f["sc"][n, b], f["q"][n, b])
    return out


def dequant_q4k_fields(f) -> np.ndarray:
    """N x K float64 w^ = d*sc*q - dmin*mn, straight from the fields."""
    N, nb = f["d"].shape
    d = f["d"].astype(np.float64)[:, :, None]
    dm = f["dmin"].astype(np.float64)[:, :, None]
    sc = np.repeat(f["sc"], 32, axis=2).astype(np.float64)
    mn = np.repeat(f["mn"], 32, axis=2).astype(np.float64)
    return (d * sc * f["q"] - dm * mn).reshape(N, nb * 256)


def dequant_q6k_fields(f) -> np.ndarray:
    N, nb = f["d"].shape
    d = f["d"].astype(np.float64)[:, :, None]
    sc = np.repeat(f["sc"], 16, axis=2).astype(np.float64)
    return (d * sc * (f["q"] - 32)).reshape(N, nb * 256)


# --- Q5_K and Q8_0 (the decoder's other block types) --------------------------

def q5k_position(i: int):
    """(qs byte, qs shift, qh byte, qh bit) of the 5-bit code of weight i."""
    c, r = divmod(i, 64)
    l = r % 32
    upper = r >= 32
    return 32 * c + l, (4 if upper else 0), l, 2 * c + (1 if upper else 0)


def enc_q5k(d: float, dmin: float, sc, mn, q) -> np.ndarray:
    """Fields -> one 176-byte Q5_K block.  sc, mn in [0,63] (Q4_K packing); q in [0,31]."""
    blk = np.zeros(176, np.uint8)
    blk[0:2] = np.array([d], np.float16).view(np.uint8)
    blk[2:4] = np.array([dmin], np.float16).view(np.uint8)
    s = np.zeros(12, np.int64)
    for j in range(8):
        sp, mp = q4k_scale_bits(j)
        for (byte, shift, width, vshift) in sp:
            s[byte] |= ((int(sc[j]) >> vshift) & ((1 << width) - 1)) << shift
        for (byte, shift, width, vshift) in mp:
            s[byte] |= ((int(mn[j]) >> vshift) & ((1 << width) - 1)) << shift
    blk[4:16] = s.astype(np.uint8)
    qh = np.zeros(32, np.int64)
    qs = np.zeros(128, np.int64)
    for i in range(256):
        qb, qsft, hb, hbit = q5k_position(i)
        qs[qb] |= (int(q[i]) & 15) << qsft
        qh[hb] |= ((int(q[i]) >> 4) & 1) << hbit
    blk[16:48] = qh.astype(np.uint8)
    blk[48:176] = qs.astype(np.uint8)
    return blk


def enc_q8_0(d: float, q) -> np.ndarray:
    """Fields -> one 34-byte Q8_0 block: d as fp16, q int8 [32]."""
    blk = np.zeros(34, np.uint8)
    blk[0:2] = np.array([d], np.float16).view(np.uint8)
    blk[2:34] = np.asarray(q, np.int8).view(np.uint8)
    return blk


def random_q5k_fields(rng, N, nb):
    f = random_q4k_fields(rng, N, nb)
    f["q"] = rng.integers(0, 32, (N, nb, 256))
    return f


def random_q8_0_fields(rng, N, nblk32):
    d = (np.abs(rng.standard_normal((N, nblk32))) * 2e-2).astype(np.float16)
    q = rng.integers(-128, 128, (N, nblk32, 32))
    return dict(d=d, q=q)


def encode_q5k_matrix(f) -> np.ndarray:
    N, nb = f["d"].shape
    out = np.zeros((N, nb, 176), np.uint8)
    for n in range(N):
        for b in range(nb):
            out[n, b] = enc_q5k(f["d"][n, b], f["dmin"][n, b], f["sc"][n, b], f["mn"][n, b],
                                f["q"][n, b])
    return out


def encode_q8_0_matrix(f) -> np.ndarray:
    N, nb = f["d"].shape
    out = np.zeros((N, nb, 34), np.uint8)
    for n in range(N):
        for b in range(nb):
            out[n, b] = enc_q8_0(f["d"][n, b], f["q"][n, b])
    return out


def dequant_q5k_fields(f) -> np.ndarray:
    return dequant_q4k_fields(f)  # same formula, 5-bit codes


def dequant_q8_0_fields(f) -> np.ndarray:
    N, nb = f["d"].shape
    return (f["d"].astype(np.float64)[:, :, None] * f["q"]).reshape(N, nb * 32)
