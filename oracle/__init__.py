"""Scalar CPU oracle for the K-quant x int8 GEMM (test infrastructure only).

Only the test suite, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg
of ``bench.py`` may import this package.  The product path (the HIP library
and its Python binding) never does.  The arithmetic lives in ``dq_oracle.c``
(plain C, built with gcc, no fast-math); this module only marshals numpy
arrays, splits the weight rows over threads and, for ``qgemm_rows``, gathers
canvas rows by index before quantizing.

Sources (each routine in ``dq_oracle.c`` cites its own):
  * mojo-dllm "Architecture" page, "Source map": scalar K-quant decoders are
    the test oracle; int8 activations with one scale per 256 values; a
    row-major reference GEMM.
  * same page, "A forward pass", steps 2-4: quantize once and reuse; the
    output projection runs on the requested rows only.
  * heatdrop.ai card, "Key highlights": GEMM checked against dequantization.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

F32, F16, Q8_0, Q4_K, Q5_K, Q6_K, BF16 = 0, 1, 8, 12, 13, 14, 30  # GGUF type ids
QK = 256
BLOCK_BYTES = {Q4_K: 144, Q6_K: 210}
SUBBLOCKS = {Q4_K: 8, Q6_K: 16}

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "dq_oracle.c")
_LIB = os.path.join(_HERE, "libdq_oracle.so")
_lib = None
_lock = threading.Lock()


def build(force: bool = False) -> str:
    """Compile dq_oracle.c with gcc into oracle/libdq_oracle.so."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(
            ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off",
             "-fno-fast-math", "-Wall", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    with _lock:
        if _lib is None:
            build()
            lib = ctypes.CDLL(_LIB)
            i64, vp = ctypes.c_int64, ctypes.c_void_p
            lib.dqo_fp16_to_f32.restype = ctypes.c_float
            lib.dqo_fp16_to_f32.argtypes = [ctypes.c_uint16]
            lib.dqo_decode_q4k.argtypes = [vp] * 6
            lib.dqo_decode_q6k.argtypes = [vp] * 4
            lib.dqo_dequant_row.argtypes = [ctypes.c_int, vp, i64, vp]
            lib.dqo_quantize_act.argtypes = [i64, i64, vp, i64, vp, vp, vp]
            lib.dqo_exp_f32.restype = ctypes.c_float
            lib.dqo_exp_f32.argtypes = [ctypes.c_float]
            lib.dqo_silu_mul.restype = ctypes.c_float
            lib.dqo_silu_mul.argtypes = [ctypes.c_float, ctypes.c_float]
            lib.dqo_swiglu_quantize_act.argtypes = [i64, i64, vp, i64, vp, vp, vp]
            lib.dqo_rmsnorm_quantize_act.argtypes = [i64, i64, vp, i64, vp, ctypes.c_float,
                                                     vp, vp, vp]
            lib.dqo_subdots.argtypes = [ctypes.c_int, i64, i64, i64, vp, vp, i64, i64, vp]
            lib.dqo_superblock_sums.argtypes = [ctypes.c_int, i64, i64, i64, vp, vp, vp,
                                                i64, i64, vp, vp]
            lib.dqo_qgemm_ref.argtypes = [ctypes.c_int, i64, i64, i64, vp, vp, vp, i64, i64,
                                          vp, vp]
            lib.dqo_qgemm_ref_points.argtypes = [ctypes.c_int, i64, i64, vp, vp, vp, vp, vp,
                                                 vp, vp]
            lib.dqo_qgemm_f32.argtypes = [ctypes.c_int, i64, i64, i64, vp, vp, vp, vp, i64,
                                          i64, vp, i64]
            lib.dqo_logits_stats.argtypes = [i64, i64, vp, i64, ctypes.c_float, vp, vp]
            lib.dqo_f32_to_fp16.restype = ctypes.c_uint16
            lib.dqo_f32_to_fp16.argtypes = [ctypes.c_float]
            lib.dqo_f32_to_fp16_n.argtypes = [vp, vp, i64]
            lib.dqo_rope_pair.argtypes = [ctypes.c_float] * 4 + [vp, vp]
            lib.dqo_rope_rows.argtypes = [i64, i64, i64, vp, i64, vp, ctypes.c_int]
            lib.dqo_decode_q8_0.argtypes = [vp, vp, vp]
            lib.dqo_decode_q5k.argtypes = [vp] * 6
            lib.dqo_row_bytes.restype = i64
            lib.dqo_row_bytes.argtypes = [ctypes.c_int, i64]
            lib.dqo_decode_row.argtypes = [ctypes.c_int, vp, i64, vp]
            lib.dqo_embed_rows.argtypes = [ctypes.c_int, i64, i64, vp, vp, i64, vp, i64, vp]
            lib.dqo_attention.argtypes = [i64, i64, i64, i64, vp, i64, vp, ctypes.c_int, vp, i64,
                                          vp]
            for name in ("dqo_dequant_row", "dqo_quantize_act", "dqo_swiglu_quantize_act",
                         "dqo_rmsnorm_quantize_act", "dqo_subdots",
                         "dqo_superblock_sums", "dqo_qgemm_ref", "dqo_qgemm_ref_points",
                         "dqo_qgemm_f32", "dqo_logits_stats", "dqo_attention", "dqo_rope_rows",
                         "dqo_decode_row", "dqo_embed_rows"):
                getattr(lib, name).restype = ctypes.c_int
            _lib = lib
    return _lib


def _p(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(ctypes.c_void_p)


def _check(rc):
    if rc != 0:
        raise ValueError("oracle rejected its arguments (rc=%d)" % rc)


def _rows(W: np.ndarray, type_: int, K: int) -> np.ndarray:
    W = np.ascontiguousarray(W, dtype=np.uint8)
    nb = K // QK
    return W.reshape(-1, nb * BLOCK_BYTES[type_])


def host_threads() -> int:
    """Threads the oracle runs on: the cores this process may use, capped by
    OMP_NUM_THREADS when the environment sets it (a job's CPU share)."""
    try:
        t = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        t = os.cpu_count() or 1
    cap = os.environ.get("OMP_NUM_THREADS", "")
    if cap.isdigit() and int(cap) > 0:
        t = min(t, int(cap))
    return max(1, t)


def _threads(n: int, threads: int | None):
    t = threads or host_threads()
    t = max(1, min(t, n))
    bounds = [n * i // t for i in range(t + 1)]
    return [(bounds[i], bounds[i + 1]) for i in range(t) if bounds[i + 1] > bounds[i]]


def _run_threaded(fn, ranges):
    if len(ranges) == 1:
        fn(*ranges[0])
        return
    ts = [threading.Thread(target=fn, args=r) for r in ranges]
    for t in ts:
        t.start()
    for t in ts:
        t.join()


# --------------------------------------------------------------------------- #
# Element-level routines                                                      #
# --------------------------------------------------------------------------- #
def fp16_to_f32(bits: np.ndarray) -> np.ndarray:
    lib = _load()
    bits = np.asarray(bits, dtype=np.uint16).ravel()
    return np.array([lib.dqo_fp16_to_f32(int(b)) for b in bits], dtype=np.float32)


def decode_q4k(block: np.ndarray):
    """One 144-byte Q4_K block -> (d, dmin, sc[8], mn[8], q[256])."""
    lib = _load()
    blk = np.ascontiguousarray(block, dtype=np.uint8)
    assert blk.size == 144
    d, dm = ctypes.c_float(), ctypes.c_float()
    sc, mn, q = (np.zeros(8, np.uint8), np.zeros(8, np.uint8), np.zeros(256, np.uint8))
    lib.dqo_decode_q4k(_p(blk), ctypes.byref(d), ctypes.byref(dm), _p(sc), _p(mn), _p(q))
    return np.float32(d.value), np.float32(dm.value), sc, mn, q


def decode_q6k(block: np.ndarray):
    """One 210-byte Q6_K block -> (d, sc[16] int8, q[256] in [0, 63])."""
    lib = _load()
    blk = np.ascontiguousarray(block, dtype=np.uint8)
    assert blk.size == 210
    d = ctypes.c_float()
    sc, q = np.zeros(16, np.int8), np.zeros(256, np.uint8)
    lib.dqo_decode_q6k(_p(blk), ctypes.byref(d), _p(sc), _p(q))
    return np.float32(d.value), sc, q


def dequant(type_: int, W: np.ndarray, K: int) -> np.ndarray:
    """Fully dequantized N x K weights in float64."""
    lib = _load()
    rows = _rows(W, type_, K)
    out = np.zeros((rows.shape[0], K), np.float64)
    for n in range(rows.shape[0]):
        r = np.ascontiguousarray(rows[n])
        o = out[n]
        _check(lib.dqo_dequant_row(type_, _p(r), K, o.ctypes.data_as(ctypes.c_void_p)))
    return out


def quantize_act(x: np.ndarray):
    """f32 M x K -> (q int8 M x K, d f32 M x K/256, bsum int32 M x K/32)."""
    lib = _load()
    x = np.ascontiguousarray(x, dtype=np.float32)
    M, K = x.shape
    q = np.zeros((M, K), np.int8)
    d = np.zeros((M, K // QK), np.float32)
    bs = np.zeros((M, K // 32), np.int32)
    _check(lib.dqo_quantize_act(M, K, _p(x), K, _p(q), _p(d), _p(bs)))
    return q, d, bs


def exp_f32(t) -> np.ndarray:
    """The defined binary32 exponential used by SiLU (dq_oracle.c, dqo_exp_f32), elementwise."""
    lib = _load()
    t = np.asarray(t, dtype=np.float32)
    return np.array([lib.dqo_exp_f32(float(v)) for v in t.ravel()], np.float32).reshape(t.shape)


def silu_mul(g, u) -> np.ndarray:
    """silu(g) * u in the defined binary32 steps, elementwise (small arrays)."""
    lib = _load()
    g = np.asarray(g, dtype=np.float32)
    u = np.broadcast_to(np.asarray(u, dtype=np.float32), g.shape)
    return np.array([lib.dqo_silu_mul(float(a), float(b)) for a, b in zip(g.ravel(), u.ravel())],
                    np.float32).reshape(g.shape)


def swiglu_quantize_act(gu: np.ndarray, F: int):
    """gu f32 M x (>= 2F): [gate | up] -> quantized silu(gate) * up, as quantize_act returns."""
    lib = _load()
    gu = np.ascontiguousarray(gu, dtype=np.float32)
    M, ld = gu.shape
    q = np.zeros((M, F), np.int8)
    d = np.zeros((M, F // QK), np.float32)
    bs = np.zeros((M, F // 32), np.int32)
    _check(lib.dqo_swiglu_quantize_act(M, F, _p(gu), ld, _p(q), _p(d), _p(bs)))
    return q, d, bs


def rmsnorm_quantize_act(x: np.ndarray, gamma: np.ndarray, eps: float):
    """RMSNorm of each row of x (f32 M x K) with weight gamma (K), then quantize_act."""
    lib = _load()
    x = np.ascontiguousarray(x, dtype=np.float32)
    gamma = np.ascontiguousarray(gamma, dtype=np.float32)
    M, K = x.shape
    q = np.zeros((M, K), np.int8)
    d = np.zeros((M, K // QK), np.float32)
    bs = np.zeros((M, K // 32), np.int32)
    _check(lib.dqo_rmsnorm_quantize_act(M, K, _p(x), K, _p(gamma), float(eps), _p(q), _p(d),
                                        _p(bs)))
    return q, d, bs


def subdots(type_: int, q: np.ndarray, W: np.ndarray, N: int, threads=None) -> np.ndarray:
    """Integer dot per (m, n, super-block, sub-block): int32 [M, N, K/256, J]."""
    lib = _load()
    q = np.ascontiguousarray(q, dtype=np.int8)
    M, K = q.shape
    Wr = _rows(W, type_, K)
    J = SUBBLOCKS[type_]
    out = np.zeros((M, N, K // QK, J), np.int32)
    _run_threaded(lambda a, b: _check(lib.dqo_subdots(type_, M, N, K, _p(q), _p(Wr), a, b,
                                                        _p(out))), _threads(N, threads))
    return out


def superblock_sums(type_: int, q, bsum, W, N: int, threads=None):
    """(S, Mn) int32 [M, N, K/256]: sum_j sc_j*dot_j and sum_j mn_j*bsum_j."""
    lib = _load()
    q = np.ascontiguousarray(q, dtype=np.int8)
    bsum = np.ascontiguousarray(bsum, dtype=np.int32)
    M, K = q.shape
    Wr = _rows(W, type_, K)
    S = np.zeros((M, N, K // QK), np.int32)
    Mn = np.zeros((M, N, K // QK), np.int32)
    _run_threaded(lambda a, b: _check(lib.dqo_superblock_sums(
        type_, M, N, K, _p(q), _p(bsum), _p(Wr), a, b, _p(S), _p(Mn))), _threads(N, threads))
    return S, Mn


def qgemm_ref(type_: int, q, d, W, N: int, threads=None):
    """Plain definition in f64: (y, T), both M x N, T = sum_k |w^ x^|."""
    lib = _load()
    q = np.ascontiguousarray(q, dtype=np.int8)
    d = np.ascontiguousarray(d, dtype=np.float32)
    M, K = q.shape
    Wr = _rows(W, type_, K)
    y = np.zeros((M, N), np.float64)
    T = np.zeros((M, N), np.float64)
    _run_threaded(lambda a, b: _check(lib.dqo_qgemm_ref(type_, M, N, K, _p(q), _p(d), _p(Wr),
                                                        a, b, _p(y), _p(T))),
                  _threads(N, threads))
    return y, T


def qgemm_ref_points(type_: int, q, d, W, m_idx, n_idx, threads=None):
    """Plain-definition (y, T) at the listed (m, n) output points only."""
    lib = _load()
    q = np.ascontiguousarray(q, dtype=np.int8)
    d = np.ascontiguousarray(d, dtype=np.float32)
    M, K = q.shape
    Wr = _rows(W, type_, K)
    mi = np.ascontiguousarray(m_idx, dtype=np.int64)
    ni = np.ascontiguousarray(n_idx, dtype=np.int64)
    P = mi.size
    y = np.zeros(P, np.float64)
    T = np.zeros(P, np.float64)

    def run(a, b):
        _check(lib.dqo_qgemm_ref_points(
            type_, K, b - a, mi[a:].ctypes.data_as(ctypes.c_void_p),
            ni[a:].ctypes.data_as(ctypes.c_void_p), _p(q), _p(d), _p(Wr),
            y[a:].ctypes.data_as(ctypes.c_void_p), T[a:].ctypes.data_as(ctypes.c_void_p)))

    _run_threaded(run, _threads(P, threads))
    return y, T


def qgemm_f32(type_: int, q, d, bsum, W, N: int, threads=None):
    """Integer decomposition folded in f32 (the oracle's own f32 output)."""
    lib = _load()
    q = np.ascontiguousarray(q, dtype=np.int8)
    d = np.ascontiguousarray(d, dtype=np.float32)
    bsum = np.ascontiguousarray(bsum, dtype=np.int32)
    M, K = q.shape
    Wr = _rows(W, type_, K)
    y = np.zeros((M, N), np.float32)
    _run_threaded(lambda a, b: _check(lib.dqo_qgemm_f32(type_, M, N, K, _p(q), _p(d), _p(bsum),
                                                        _p(Wr), a, b, _p(y), N)),
                  _threads(N, threads))
    return y


def qgemm_rows_inputs(canvas: np.ndarray, idx: np.ndarray):
    """Gathered-row projection, activation side: quantize rows canvas[idx].

    Architecture page, "A forward pass", steps 3-4: only the requested
    positions reach the output projection.  Returns (q, d, bsum) of the
    gathered rows in idx order (duplicates allowed).
    """
    rows = np.ascontiguousarray(np.asarray(canvas, np.float32)[np.asarray(idx, np.int64)])
    return quantize_act(rows)


def logits_stats(y: np.ndarray, beta: float = 1.0):
    """Sampler statistics of each row of a logits matrix (dqo_logits_stats).

    heatdrop.ai card, "The interesting bit", and the aiboss88 news page's
    capability list: the samplers read the requested rows' logits (LLaDA ranks
    by the confidence of its greedy prediction, Dream by entropy).  With
    z = beta * y (binary32): returns (token int32[M], stats float64[M, 4]) where
    stats[m] = (max z, log sum exp z, entropy of softmax z, softmax probability
    of the token) and token is the first index of the maximum.
    """
    y = np.ascontiguousarray(np.atleast_2d(np.asarray(y, np.float64)))
    M, N = y.shape
    token = np.zeros(M, np.int32)
    stats = np.zeros((M, 4), np.float64)
    _check(_load().dqo_logits_stats(M, N, _p(y), N, ctypes.c_float(beta), _p(token), _p(stats)))
    return token, stats


def qgemm_rows_sample_ref(type_: int, canvas: np.ndarray, idx: np.ndarray, W, N: int,
                          beta: float = 1.0, threads=None):
    """Gathered-row projection followed by the sampler statistics of its rows.

    Returns (token, stats, y, T): the statistics of the plain-definition logits
    y (f64, M x N) of the rows canvas[idx], and the tolerance scale T of y.
    """
    q, d, _ = qgemm_rows_inputs(canvas, idx)
    y, T = qgemm_ref(type_, q, d, W, N, threads)
    token, stats = logits_stats(y, beta)
    return token, stats, y, T


# --- attention over the canvas ------------------------------------------------

ROPE_NONE, ROPE_NORM, ROPE_NEOX = 0, 1, 2


def f32_to_fp16_bits(x: np.ndarray) -> np.ndarray:
    """IEEE binary32 -> binary16 (round to nearest even), as uint16 bit patterns."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    h = np.zeros(x.shape, np.uint16)
    _load().dqo_f32_to_fp16_n(_p(x), _p(h), x.size)
    return h


def rope_pair(a: float, b: float, c: float, s: float):
    """One RoPE rotation of the pair (a, b) by (cos, sin) = (c, s), in binary32."""
    ra, rb = ctypes.c_float(), ctypes.c_float()
    _load().dqo_rope_pair(a, b, c, s, ctypes.byref(ra), ctypes.byref(rb))
    return ra.value, rb.value


def rope_rows(x: np.ndarray, n_heads: int, D: int, rope: np.ndarray, mode: int) -> np.ndarray:
    """RoPE of the n_heads head vectors of each row (row l at position l): a copy."""
    x = np.array(x, dtype=np.float32, order="C", copy=True)
    rope = np.ascontiguousarray(rope, dtype=np.float32)
    _check(_load().dqo_rope_rows(x.shape[0], n_heads, D, _p(x), x.shape[1], _p(rope), mode))
    return x


def attention(qkv: np.ndarray, H: int, Hkv: int, D: int, rope=None, mode: int = ROPE_NONE):
    """Bidirectional attention of every canvas position over all L positions.

    Architecture page, "A forward pass", step 2 (RoPE on Q and K, attention over
    all L positions, no mask) and "Source map" (NORM and NEOX RoPE); aiboss88 news
    page, capability list (attention on f16 tensor cores).  qkv: L x ((H + 2 Hkv) D)
    f32 rows [Q | K | V]; rope: L x D/2 x 2 (cos, sin) f32 or None.  Q and K are
    rotated in binary32, Q, K and V rounded to binary16, the rest is binary64.
    Returns (out [L, H D], tol [L, H D]) with tol = sum_j p_j |v_j| / sum_j p_j.
    """
    qkv = np.ascontiguousarray(qkv, dtype=np.float32)
    L = qkv.shape[0]
    if rope is not None:
        rope = np.ascontiguousarray(rope, dtype=np.float32)
    out = np.zeros((L, H * D), np.float64)
    tol = np.zeros((L, H * D), np.float64)
    _check(_load().dqo_attention(L, H, Hkv, D, _p(qkv), qkv.shape[1],
                                 _p(rope) if rope is not None else None, mode, _p(out), H * D,
                                 _p(tol)))
    return out, tol


# --- the decoder's other block types and embedding rows ----------------------

def row_bytes(type_: int, K: int) -> int:
    """Bytes of one row of K values of a GGUF type (0: unknown type or bad K)."""
    return int(_load().dqo_row_bytes(type_, K))


def decode_q8_0(block: np.ndarray):
    """34-byte Q8_0 block -> (d, q[32] int8)."""
    block = np.ascontiguousarray(block, dtype=np.uint8)
    d = ctypes.c_float()
    q = np.zeros(32, np.int8)
    _load().dqo_decode_q8_0(_p(block), ctypes.byref(d), _p(q))
    return d.value, q


def decode_q5k(block: np.ndarray):
    """176-byte Q5_K block -> (d, dmin, sc[8], mn[8], q[256] in [0, 31])."""
    block = np.ascontiguousarray(block, dtype=np.uint8)
    d, dm = ctypes.c_float(), ctypes.c_float()
    sc, mn, q = np.zeros(8, np.uint8), np.zeros(8, np.uint8), np.zeros(256, np.uint8)
    _load().dqo_decode_q5k(_p(block), ctypes.byref(d), ctypes.byref(dm), _p(sc), _p(mn), _p(q))
    return d.value, dm.value, sc, mn, q


def decode_row(type_: int, row: np.ndarray, K: int) -> np.ndarray:
    """One row of any supported GGUF type -> K float64 values (exact)."""
    row = np.ascontiguousarray(row, dtype=np.uint8).reshape(-1)
    w = np.zeros(K, np.float64)
    _check(_load().dqo_decode_row(type_, _p(row), K, _p(w)))
    return w


def embed_rows(type_: int, table: np.ndarray, K: int, ids: np.ndarray):
    """Rows ids of an N x K table in GGUF bytes (N rows of row_bytes(type, K)),
    decoded to float32 (Architecture page, "A forward pass", step 1).  Returns
    (out [M, K] float32, flag [M] int32: 1 where the id is outside [0, N))."""
    rb = row_bytes(type_, K)
    table = np.ascontiguousarray(table, dtype=np.uint8).reshape(-1)
    N = table.size // rb if rb else 0
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    M = ids.size
    out = np.zeros((M, K), np.float32)
    flag = np.zeros(M, np.int32)
    _check(_load().dqo_embed_rows(type_, N, K, _p(table), _p(ids), M, _p(out), K, _p(flag)))
    return out, flag
