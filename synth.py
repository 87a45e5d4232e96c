"""Seeded synthetic inputs for the K-quant x int8 GEMM (shared by tests and bench).

This module draws random numbers and places them at the byte offsets of the
GGUF K-quant super-blocks; it holds none of the method's arithmetic (no
decoding, quantization or products).  Both the CPU oracle and the HIP path
consume what it produces.

Draws (numpy ``default_rng(seed)``, PCG64), in this order per matrix:
  * Q4_K block (144 bytes): d then dmin as fp16(|N(0,1)| * 2e-3) at bytes 0-1
    and 2-3; the 12 scale bytes uniform on [0, 255] (the 6-bit scale/min
    packing is a bijection between these 96 bits and sixteen 6-bit values, so
    every scale and min is uniform on [0, 63]); the 128 nibble bytes uniform
    (every 4-bit code uniform on [0, 15]).
  * Q6_K block (210 bytes): d as fp16(|N(0,1)| * 2e-3) at bytes 208-209; the
    16 int8 scales at bytes 192-207 uniform on [-32, 31]; the 128 low-nibble
    bytes and 64 high-bit bytes uniform (every 6-bit code uniform on [0, 63]).
  * Activations: N(0, 1) float32, then round(0.01 * K) columns drawn without
    replacement and multiplied by 20 in every row.
  * Edge-case option (tests only): ``mixed_scales`` draws d (and dmin) as a
    mixture of positive, negative, signed-zero and subnormal fp16 values.
"""
from __future__ import annotations

import numpy as np

Q4_K = 12
Q6_K = 14
QK = 256
BLOCK_BYTES = {Q4_K: 144, Q6_K: 210}


def _fp16_bytes(rng: np.random.Generator, shape, scale: float, mixed: bool = False) -> np.ndarray:
    """fp16 scale fields: |N(0,1)| * scale, or with ``mixed`` a mixture of
    signs and special values (the format allows any fp16 here): 35% positive
    and 35% negative normal values of that size, 10% signed zeros, 20% random
    subnormal patterns of either sign."""
    v = (np.abs(rng.standard_normal(shape)) * scale).astype(np.float16)
    if mixed:
        bits = v.view(np.uint16).copy()
        u = rng.random(shape)
        sign = rng.integers(0, 2, shape).astype(np.uint16) << 15
        sub = rng.integers(1, 1024, shape).astype(np.uint16)
        bits = np.where(u < 0.35, bits, bits | np.uint16(0x8000))
        bits = np.where((u >= 0.70) & (u < 0.80), sign, bits)
        bits = np.where(u >= 0.80, sign | sub, bits)
        v = bits.astype(np.uint16).view(np.float16)
    return v.view(np.uint8).reshape(tuple(shape) + (2,))


def _bytes(rng: np.random.Generator, shape) -> np.ndarray:
    n = int(np.prod(shape))
    return np.frombuffer(rng.bytes(n), dtype=np.uint8).reshape(shape)


def q4k_weights(rng: np.random.Generator, N: int, K: int, d_scale: float = 2e-3,
                mixed_scales: bool = False) -> np.ndarray:
    """N x K weights as raw Q4_K blocks, uint8 [N, K/256, 144].  With
    ``mixed_scales`` d and dmin take signs, zeros and subnormals too."""
    nb = K // QK
    out = np.empty((N, nb, 144), np.uint8)
    out[..., 0:2] = _fp16_bytes(rng, (N, nb), d_scale, mixed_scales)
    out[..., 2:4] = _fp16_bytes(rng, (N, nb), d_scale, mixed_scales)
    out[..., 4:16] = _bytes(rng, (N, nb, 12))
    out[..., 16:144] = _bytes(rng, (N, nb, 128))
    return out


def q6k_weights(rng: np.random.Generator, N: int, K: int, d_scale: float = 2e-3,
                sc_lo: int = -32, sc_hi: int = 31, mixed_scales: bool = False) -> np.ndarray:
    """N x K weights as raw Q6_K blocks, uint8 [N, K/256, 210].  With
    ``mixed_scales`` d takes signs, zeros and subnormals too."""
    nb = K // QK
    out = np.empty((N, nb, 210), np.uint8)
    out[..., 208:210] = _fp16_bytes(rng, (N, nb), d_scale, mixed_scales)
    out[..., 192:208] = rng.integers(sc_lo, sc_hi + 1, size=(N, nb, 16)).astype(np.int8).view(
        np.uint8)
    out[..., 0:192] = _bytes(rng, (N, nb, 192))
    return out


def weights(rng: np.random.Generator, type_: int, N: int, K: int) -> np.ndarray:
    return q4k_weights(rng, N, K) if type_ == Q4_K else q6k_weights(rng, N, K)


def activations(rng: np.random.Generator, M: int, K: int, outlier_frac: float = 0.01,
                outlier_mul: float = 20.0) -> np.ndarray:
    """M x K float32 ~ N(0,1) with round(outlier_frac*K) columns scaled by outlier_mul."""
    x = rng.standard_normal((M, K), dtype=np.float32)
    n_out = int(round(outlier_frac * K))
    if n_out:
        cols = rng.choice(K, size=n_out, replace=False)
        x[:, cols] *= np.float32(outlier_mul)
    return x


def row_index(rng: np.random.Generator, L: int, M: int) -> np.ndarray:
    """M distinct canvas rows of [0, L), sorted ascending, int32."""
    return np.sort(rng.choice(L, size=M, replace=False)).astype(np.int32)


# --------------------------------------------------------------------------- #
# Workloads (shapes of the five configurations; seeds 1000*config+10*layer+p)  #
# --------------------------------------------------------------------------- #
LLADA = dict(L=160, K=4096, ffn=12288, vocab=126464, layers=32, heads=32, kv_heads=32,
             head_dim=128, rope_theta=500000.0, rope="norm")
DREAM = dict(L=512, K=3584, ffn=18944, kv=512, vocab=152064, heads=28, kv_heads=4,
             head_dim=128, rope_theta=1000000.0, rope="neox")


def llada_layer(layer: int):
    """(name, type, N, K) of one LLaDA-8B layer's projections.

    Down is Q6_K on odd layers and Q4_K on even layers.
    """
    K, F = LLADA["K"], LLADA["ffn"]
    down_t = Q6_K if layer % 2 else Q4_K
    return [("q", Q4_K, K, K), ("k", Q4_K, K, K), ("v", Q4_K, K, K), ("o", Q4_K, K, K),
            ("gate", Q4_K, F, K), ("up", Q4_K, F, K), ("down", down_t, K, F)]


def dream_layer():
    K, F, KV = DREAM["K"], DREAM["ffn"], DREAM["kv"]
    return [("q", Q4_K, K, K), ("k", Q4_K, KV, K), ("v", Q4_K, KV, K), ("o", Q4_K, K, K),
            ("gate", Q4_K, F, K), ("up", Q4_K, F, K), ("down", Q6_K, K, F)]


def seed(config: int, layer: int, proj: int) -> int:
    return 1000 * config + 10 * layer + proj


def rope_table(L: int, D: int, theta: float) -> np.ndarray:
    """L x D/2 x 2 float32 (cos, sin) of the angles pos * theta**(-2i/D), i < D/2.

    A model constant (precomputed once for the longest canvas); attention takes
    it as an input, like the RMSNorm weights.
    """
    inv = theta ** (-np.arange(0, D, 2, dtype=np.float64) / D)
    ang = np.arange(L, dtype=np.float64)[:, None] * inv[None, :]
    return np.stack([np.cos(ang), np.sin(ang)], axis=-1).astype(np.float32)


def qkv_rows(rng: np.random.Generator, L: int, H: int, Hkv: int, D: int,
             scale: float = 1.0) -> np.ndarray:
    """L x (H + 2 Hkv) D float32 rows [Q | K | V] ~ N(0, scale^2)."""
    return (rng.standard_normal((L, (H + 2 * Hkv) * D)) * scale).astype(np.float32)


# --------------------------------------------------------------------------- #
# Tables of the decoder's other GGUF types (embedding rows), raw bytes        #
# --------------------------------------------------------------------------- #
F32, F16, Q8_0, Q5_K, BF16 = 0, 1, 8, 13, 30


def q5k_weights(rng: np.random.Generator, N: int, K: int, d_scale: float = 2e-3) -> np.ndarray:
    """N x K as raw Q5_K blocks, uint8 [N, K/256, 176]: d, dmin as in Q4_K, then
    the 12 scale bytes, 32 fifth-bit bytes and 128 nibble bytes uniform."""
    nb = K // QK
    out = np.empty((N, nb, 176), np.uint8)
    out[..., 0:2] = _fp16_bytes(rng, (N, nb), d_scale)
    out[..., 2:4] = _fp16_bytes(rng, (N, nb), d_scale)
    out[..., 4:176] = _bytes(rng, (N, nb, 172))
    return out


def q8_0_weights(rng: np.random.Generator, N: int, K: int, d_scale: float = 2e-2) -> np.ndarray:
    """N x K as raw Q8_0 blocks, uint8 [N, K/32, 34]: d as fp16(|N(0,1)| d_scale),
    then 32 uniform int8 codes."""
    nb = K // 32
    out = np.empty((N, nb, 34), np.uint8)
    out[..., 0:2] = _fp16_bytes(rng, (N, nb), d_scale)
    out[..., 2:34] = _bytes(rng, (N, nb, 32))
    return out


def float_table(rng: np.random.Generator, type_: int, N: int, K: int) -> np.ndarray:
    """N x K N(0,1) values as raw F32, F16 or BF16 bytes (BF16: the top half of
    each binary32 pattern), uint8 [N, bytes per row]."""
    x = rng.standard_normal((N, K)).astype(np.float32)
    if type_ == F32:
        return x.view(np.uint8).reshape(N, 4 * K)
    if type_ == F16:
        return x.astype(np.float16).view(np.uint8).reshape(N, 2 * K)
    return (x.view(np.uint32) >> 16).astype(np.uint16).view(np.uint8).reshape(N, 2 * K)


def table(rng: np.random.Generator, type_: int, N: int, K: int) -> np.ndarray:
    """A random N x K table of any decoded GGUF type, as raw bytes [N, row bytes]."""
    gen = {Q4_K: q4k_weights, Q6_K: q6k_weights, Q5_K: q5k_weights, Q8_0: q8_0_weights}
    if type_ in gen:
        return gen[type_](rng, N, K).reshape(N, -1)
    return float_table(rng, type_, N, K)
