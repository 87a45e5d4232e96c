"""Python binding of libdq (include/dq.h): the GGUF K-quant x int8 GEMM on MI355X.

Argument marshalling only: every step runs in the HIP kernels of libdq.so,
which must have been built in-tree (``__graft_entry__.build()`` or
``python quantized_gemm_diffusion_amd/_build.py``).  There is no fallback: if
the library is missing, every call raises.  torch supplies device memory and
the current stream; tensors must live on a GPU.

Names follow the C ABI:
  packed_size, repack_weights, act_size, quantize_act, swiglu_quantize_act,
  rmsnorm_quantize_act, qgemm, qgemm_rows_workspace, qgemm_rows, qgemm_rows_noalloc,
  debug_superblock_sums, ...
Quantized activations travel as an ``Act`` (the device buffer in the record
layout that include/dq.h documents, with its M and K).
"""
from __future__ import annotations

import ctypes
import os
import threading
from typing import NamedTuple

import torch

Q4_K = 12
Q6_K = 14
QK = 256
BLOCK_BYTES = {Q4_K: 144, Q6_K: 210}

DQ_OK, DQ_EINVAL, DQ_EUNSUPPORTED, DQ_EWORKSPACE, DQ_EHIP = 0, 1, 2, 3, 4

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libdq.so")

EXPORTS = ("dq_status_string", "dq_last_error", "dq_packed_size", "dq_repack_weights",
           "dq_act_size", "dq_quantize_act", "dq_swiglu_quantize_act", "dq_rmsnorm_quantize_act",
           "dq_qgemm", "dq_qgemm_swiglu", "dq_qgemm_rows_workspace", "dq_qgemm_rows", "dq_qgemm_rows_noalloc",
           "dq_logits_stats_workspace",
           "dq_logits_stats", "dq_qgemm_rows_sample_workspace", "dq_qgemm_rows_sample",
           "dq_attention_workspace", "dq_attention", "dq_row_bytes", "dq_embed_rows",
           "dq_debug_superblock_sums", "dq_debug_subdots")
ACT_RECORD = 5120  # bytes per (super-block, 16-row block) record


class Act(NamedTuple):
    """Quantized activations: ``buf`` (uint8, act_size(M, K) bytes) for M rows of K."""
    buf: torch.Tensor
    M: int
    K: int


_lib = None
_lock = threading.Lock()


class DQError(RuntimeError):
    def __init__(self, status: int, where: str, msg: str):
        super().__init__(f"{where}: {msg} (status {status})")
        self.status = status


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libdq.so and declare the C signatures.  Raises if it is not built."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is not built; run __graft_entry__.build() first")
        lib = ctypes.CDLL(path)
        i32, i64, vp, sz = ctypes.c_int, ctypes.c_int64, ctypes.c_void_p, ctypes.c_size_t
        psz = ctypes.POINTER(ctypes.c_size_t)
        lib.dq_status_string.restype = ctypes.c_char_p
        lib.dq_status_string.argtypes = [i32]
        lib.dq_last_error.restype = ctypes.c_char_p
        lib.dq_last_error.argtypes = []
        sigs = {
            "dq_packed_size": [i32, i64, i64, psz],
            "dq_repack_weights": [i32, i64, i64, vp, vp, vp],
            "dq_act_size": [i64, i64, psz],
            "dq_quantize_act": [i64, i64, vp, i64, vp, vp],
            "dq_swiglu_quantize_act": [i64, i64, vp, i64, vp, vp],
            "dq_rmsnorm_quantize_act": [i64, i64, vp, i64, vp, ctypes.c_float, vp, vp],
            "dq_qgemm": [i32, i64, i64, i64, vp, vp, vp, i64, vp],
            "dq_qgemm_swiglu": [i32, i64, i64, i64, vp, vp, vp, i64, vp],
            "dq_debug_subdots": [i32, i64, i64, i64, vp, vp, vp, vp],
            "dq_qgemm_rows_workspace": [i64, i64, psz],
            "dq_qgemm_rows": [i32, i64, i64, i64, i64, vp, i64, vp, vp, vp, i64, vp, sz, vp],
            "dq_qgemm_rows_noalloc": [i32, i64, i64, i64, i64, vp, i64, vp, vp, vp, i64, vp, vp],
            "dq_logits_stats_workspace": [i64, i64, psz],
            "dq_logits_stats": [i64, i64, vp, i64, ctypes.c_float, vp, vp, vp, sz, vp],
            "dq_qgemm_rows_sample_workspace": [i64, i64, i64, psz],
            "dq_qgemm_rows_sample": [i32, i64, i64, i64, i64, vp, i64, vp, vp, ctypes.c_float, vp,
                                     vp, vp, sz, vp],
            "dq_attention_workspace": [i64, i64, i64, i64, psz],
            "dq_attention": [i64, i64, i64, i64, vp, i64, vp, i32, vp, i64, vp, sz, vp],
            "dq_row_bytes": [i32, i64, psz],
            "dq_embed_rows": [i32, i64, i64, vp, vp, i64, vp, i64, vp, vp],
            "dq_debug_superblock_sums": [i32, i64, i64, i64, vp, vp, vp, vp, vp],
        }
        for name, args in sigs.items():
            fn = getattr(lib, name)
            fn.restype = i32
            fn.argtypes = args
        _lib = lib
        return lib


def _check(status: int, where: str):
    if status != DQ_OK:
        lib = load_library()
        raise DQError(status, where, lib.dq_last_error().decode())


def _ptr(t) -> int | None:
    return None if t is None else t.data_ptr()


def _stream(t: torch.Tensor) -> int:
    if not t.is_cuda:
        raise ValueError("libdq works on GPU tensors only")
    return torch.cuda.current_stream(t.device).cuda_stream


def _need(t: torch.Tensor, dtype, name: str):
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")


def packed_size(type_: int, N: int, K: int) -> int:
    lib = load_library()
    out = ctypes.c_size_t()
    _check(lib.dq_packed_size(type_, N, K, ctypes.byref(out)), "dq_packed_size")
    return out.value


def repack_weights(type_: int, N: int, K: int, gguf: torch.Tensor,
                   packed: torch.Tensor | None = None) -> torch.Tensor:
    """GGUF blocks (uint8, N*(K/256)*block bytes, on the GPU) -> packed tiles."""
    lib = load_library()
    _need(gguf, torch.uint8, "gguf")
    if not gguf.is_contiguous() or gguf.numel() != N * (K // QK) * BLOCK_BYTES.get(type_, 0):
        raise ValueError("gguf must be contiguous with N*(K/256) blocks of the given type")
    if packed is None:
        packed = torch.empty(packed_size(type_, N, K), dtype=torch.uint8, device=gguf.device)
    _need(packed, torch.uint8, "packed")
    _check(lib.dq_repack_weights(type_, N, K, _ptr(gguf), _ptr(packed), _stream(gguf)),
           "dq_repack_weights")
    return packed


def act_size(M: int, K: int) -> int:
    lib = load_library()
    out = ctypes.c_size_t()
    _check(lib.dq_act_size(M, K, ctypes.byref(out)), "dq_act_size")
    return out.value


def quantize_act(x: torch.Tensor, out: torch.Tensor | None = None) -> Act:
    """f32 [M, K] (row stride >= K, unit column stride) -> Act."""
    lib = load_library()
    _need(x, torch.float32, "x")
    if x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be 2-D with unit column stride")
    M, K = x.shape
    nbytes = act_size(M, K)
    if out is None:
        out = torch.empty(nbytes, dtype=torch.uint8, device=x.device)
    _need(out, torch.uint8, "out")
    if out.numel() < nbytes or not out.is_contiguous():
        raise ValueError(f"out must be a contiguous buffer of at least {nbytes} bytes")
    _check(lib.dq_quantize_act(M, K, _ptr(x), x.stride(0) if M > 1 else K, _ptr(out),
                               _stream(x)), "dq_quantize_act")
    return Act(out, M, K)


def _act_out(M: int, K: int, out, dev):
    nbytes = act_size(M, K)
    if out is None:
        out = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    _need(out, torch.uint8, "out")
    if out.numel() < nbytes or not out.is_contiguous():
        raise ValueError(f"out must be a contiguous buffer of at least {nbytes} bytes")
    return out


def swiglu_quantize_act(gu: torch.Tensor, F: int, out: torch.Tensor | None = None) -> Act:
    """f32 [M, >= 2F] rows of [gate | up] -> Act of silu(gate) * up (M x F)."""
    lib = load_library()
    _need(gu, torch.float32, "gu")
    if gu.dim() != 2 or gu.stride(1) != 1 or gu.shape[1] < 2 * F:
        raise ValueError("gu must be 2-D [M, >= 2F] with unit column stride")
    M = gu.shape[0]
    out = _act_out(M, F, out, gu.device)
    _check(lib.dq_swiglu_quantize_act(M, F, _ptr(gu), gu.stride(0) if M > 1 else 2 * F,
                                      _ptr(out), _stream(gu)), "dq_swiglu_quantize_act")
    return Act(out, M, F)


def rmsnorm_quantize_act(x: torch.Tensor, gamma: torch.Tensor, eps: float,
                         out: torch.Tensor | None = None) -> Act:
    """f32 [M, K] -> Act of RMSNorm(x) * gamma."""
    lib = load_library()
    _need(x, torch.float32, "x")
    _need(gamma, torch.float32, "gamma")
    if x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be 2-D with unit column stride")
    M, K = x.shape
    if gamma.numel() != K or not gamma.is_contiguous():
        raise ValueError("gamma must be a contiguous vector of K weights")
    out = _act_out(M, K, out, x.device)
    _check(lib.dq_rmsnorm_quantize_act(M, K, _ptr(x), x.stride(0) if M > 1 else K, _ptr(gamma),
                                       float(eps), _ptr(out), _stream(x)),
           "dq_rmsnorm_quantize_act")
    return Act(out, M, K)


def _check_operands(type_, act: Act, packed, N):
    """Size checks that keep every kernel access inside the tensors."""
    _need(act.buf, torch.uint8, "act.buf")
    if act.buf.numel() < act_size(act.M, act.K) or not act.buf.is_contiguous():
        raise ValueError("act.buf is smaller than act_size(M, K)")
    _need(packed, torch.uint8, "packed")
    if packed.numel() < packed_size(type_, N, act.K) or not packed.is_contiguous():
        raise ValueError("packed is smaller than packed_size(type, N, K)")
    return act.M, act.K


def qgemm(type_: int, act: Act, packed: torch.Tensor, N: int,
          y: torch.Tensor | None = None) -> torch.Tensor:
    """y [M, N] f32 = dequant(act) @ dequant(packed)^T."""
    lib = load_library()
    M, K = _check_operands(type_, act, packed, N)
    if y is None:
        y = torch.empty((M, N), dtype=torch.float32, device=act.buf.device)
    _need(y, torch.float32, "y")
    if y.dim() != 2 or y.shape[0] != M or y.shape[1] < N or y.stride(1) != 1:
        raise ValueError("y must be [M, >=N] with unit column stride")
    _check(lib.dq_qgemm(type_, M, N, K, _ptr(act.buf), _ptr(packed), _ptr(y),
                        y.stride(0) if M > 1 else N, _stream(act.buf)), "dq_qgemm")
    return y


def qgemm_swiglu(type_: int, act: Act, packed: torch.Tensor, F: int,
                 h: torch.Tensor | None = None) -> torch.Tensor:
    """h [M, F] f32 = silu(gate) * up of the interleaved gate/up GEMM (dq.h)."""
    lib = load_library()
    M, K = _check_operands(type_, act, packed, 2 * F)
    if h is None:
        h = torch.empty((M, F), dtype=torch.float32, device=act.buf.device)
    _need(h, torch.float32, "h")
    if h.dim() != 2 or h.shape[0] != M or h.shape[1] < F or h.stride(1) != 1:
        raise ValueError("h must be [M, >=F] with unit column stride")
    _check(lib.dq_qgemm_swiglu(type_, M, F, K, _ptr(act.buf), _ptr(packed), _ptr(h),
                               h.stride(0) if M > 1 else F, _stream(act.buf)), "dq_qgemm_swiglu")
    return h


def interleave_gate_up(gate, up, rows: int = 16):
    """Stack gate and up (N = F rows each, any row type) with their 16-row
    tiles interleaved, the weight order dq_qgemm_swiglu takes: rows 32i ..
    32i+15 from gate, 32i+16 .. 32i+31 from up.  numpy or torch, along dim 0."""
    F = gate.shape[0]
    if up.shape != gate.shape or F % rows:
        raise ValueError("gate and up must have the same shape and a multiple of 16 rows")
    g = gate.reshape((F // rows, rows) + tuple(gate.shape[1:]))
    u = up.reshape((F // rows, rows) + tuple(up.shape[1:]))
    if isinstance(gate, torch.Tensor):
        return torch.stack([g, u], 1).reshape((2 * F,) + tuple(gate.shape[1:]))
    import numpy as _np
    return _np.stack([g, u], 1).reshape((2 * F,) + tuple(gate.shape[1:]))


def qgemm_rows_workspace(M: int, K: int) -> int:
    lib = load_library()
    out = ctypes.c_size_t()
    _check(lib.dq_qgemm_rows_workspace(M, K, ctypes.byref(out)), "dq_qgemm_rows_workspace")
    return out.value


def qgemm_rows(type_: int, canvas: torch.Tensor, idx: torch.Tensor, packed: torch.Tensor,
               N: int, y: torch.Tensor | None = None, ws: torch.Tensor | None = None):
    """Logits for canvas rows idx only: y [M, N] f32."""
    lib = load_library()
    _need(canvas, torch.float32, "canvas")
    _need(idx, torch.int32, "idx")
    if canvas.dim() != 2 or canvas.stride(1) != 1:
        raise ValueError("canvas must be 2-D with unit column stride")
    L, K = canvas.shape
    M = idx.numel()
    if not idx.is_contiguous():
        raise ValueError("idx must be contiguous")
    _need(packed, torch.uint8, "packed")
    if packed.numel() < packed_size(type_, N, K) or not packed.is_contiguous():
        raise ValueError("packed is smaller than packed_size(type, N, K)")
    dev = canvas.device
    if y is None:
        y = torch.empty((M, N), dtype=torch.float32, device=dev)
    if ws is None:
        ws = torch.empty(qgemm_rows_workspace(M, K), dtype=torch.uint8, device=dev)
    _need(y, torch.float32, "y")
    if y.dim() != 2 or y.shape[0] != M or y.shape[1] < N or y.stride(1) != 1:
        raise ValueError("y must be [M, >=N] with unit column stride")
    _need(ws, torch.uint8, "ws")
    _check(lib.dq_qgemm_rows(type_, L, M, N, K, _ptr(canvas), canvas.stride(0) if L > 1 else K,
                             _ptr(idx), _ptr(packed), _ptr(y),
                             y.stride(0) if M > 1 else N, _ptr(ws),
                             ws.numel() * ws.element_size(), _stream(canvas)), "dq_qgemm_rows")
    return y, ws


NOALLOC_SCRATCH_BYTES = 4194304  # DQ_NOALLOC_SCRATCH_BYTES


def qgemm_rows_noalloc(type_: int, canvas: torch.Tensor, idx: torch.Tensor, packed: torch.Tensor,
                       N: int, y: torch.Tensor, flags: torch.Tensor | None = None):
    """qgemm_rows with the workspace in the library's built-in device array
    (dq_qgemm_rows_noalloc): y [M, >=N] f32 and the optional flags [M] int32
    are caller memory; the call itself allocates nothing."""
    lib = load_library()
    _need(canvas, torch.float32, "canvas")
    _need(idx, torch.int32, "idx")
    _need(y, torch.float32, "y")
    _need(packed, torch.uint8, "packed")
    if canvas.dim() != 2 or canvas.stride(1) != 1:
        raise ValueError("canvas must be 2-D with unit column stride")
    L, K = canvas.shape
    M = idx.numel()
    if not idx.is_contiguous():
        raise ValueError("idx must be contiguous")
    if y.dim() != 2 or y.shape[0] != M or y.shape[1] < N or y.stride(1) != 1:
        raise ValueError("y must be [M, >=N] with unit column stride")
    if flags is not None:
        _need(flags, torch.int32, "flags")
        if flags.numel() < M or not flags.is_contiguous():
            raise ValueError("flags must be a contiguous int32 tensor of at least M entries")
    _check(lib.dq_qgemm_rows_noalloc(type_, L, M, N, K, _ptr(canvas),
                                     canvas.stride(0) if L > 1 else K, _ptr(idx), _ptr(packed),
                                     _ptr(y), y.stride(0) if M > 1 else N, _ptr(flags),
                                     _stream(canvas)), "dq_qgemm_rows_noalloc")
    return y


def _stats_out(M: int, token, stats, dev):
    if token is None:
        token = torch.empty(M, dtype=torch.int32, device=dev)
    if stats is None:
        stats = torch.empty((M, 4), dtype=torch.float32, device=dev)
    _need(token, torch.int32, "token")
    _need(stats, torch.float32, "stats")
    if token.numel() < M or not token.is_contiguous():
        raise ValueError("token must be a contiguous int32 tensor of at least M entries")
    if stats.numel() < 4 * M or not stats.is_contiguous():
        raise ValueError("stats must be a contiguous f32 tensor of at least 4 M entries")
    return token, stats


def _ws(nbytes: int, ws, dev):
    if ws is None:
        ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev)
    _need(ws, torch.uint8, "ws")
    return ws


def logits_stats_workspace(M: int, N: int) -> int:
    lib = load_library()
    out = ctypes.c_size_t()
    _check(lib.dq_logits_stats_workspace(M, N, ctypes.byref(out)), "dq_logits_stats_workspace")
    return out.value


def logits_stats(y: torch.Tensor, beta: float = 1.0, token=None, stats=None, ws=None):
    """Sampler statistics of each row of f32 logits y [M, N]: (token int32 [M],
    stats f32 [M, 4] = max, log-partition, entropy, top probability of
    softmax(beta * y)), ws."""
    lib = load_library()
    _need(y, torch.float32, "y")
    if y.dim() != 2 or y.stride(1) != 1:
        raise ValueError("y must be 2-D with unit column stride")
    M, N = y.shape
    token, stats = _stats_out(M, token, stats, y.device)
    ws = _ws(logits_stats_workspace(M, N), ws, y.device)
    _check(lib.dq_logits_stats(M, N, _ptr(y), y.stride(0) if M > 1 else N, beta, _ptr(token),
                               _ptr(stats), _ptr(ws), ws.numel(), _stream(y)), "dq_logits_stats")
    return token, stats, ws


def qgemm_rows_sample_workspace(M: int, N: int, K: int) -> int:
    lib = load_library()
    out = ctypes.c_size_t()
    _check(lib.dq_qgemm_rows_sample_workspace(M, N, K, ctypes.byref(out)),
           "dq_qgemm_rows_sample_workspace")
    return out.value


def qgemm_rows_sample(type_: int, canvas: torch.Tensor, idx: torch.Tensor, packed: torch.Tensor,
                      N: int, beta: float = 1.0, token=None, stats=None, ws=None):
    """The output projection on canvas rows idx with the sampler statistics
    formed in its epilogue (no logits are stored): (token, stats, ws) as for
    logits_stats."""
    lib = load_library()
    _need(canvas, torch.float32, "canvas")
    _need(idx, torch.int32, "idx")
    if canvas.dim() != 2 or canvas.stride(1) != 1:
        raise ValueError("canvas must be 2-D with unit column stride")
    L, K = canvas.shape
    M = idx.numel()
    if not idx.is_contiguous():
        raise ValueError("idx must be contiguous")
    _need(packed, torch.uint8, "packed")
    if packed.numel() < packed_size(type_, N, K) or not packed.is_contiguous():
        raise ValueError("packed is smaller than packed_size(type, N, K)")
    dev = canvas.device
    token, stats = _stats_out(M, token, stats, dev)
    ws = _ws(qgemm_rows_sample_workspace(M, N, K), ws, dev)
    _check(lib.dq_qgemm_rows_sample(type_, L, M, N, K, _ptr(canvas),
                                    canvas.stride(0) if L > 1 else K, _ptr(idx), _ptr(packed),
                                    beta, _ptr(token), _ptr(stats), _ptr(ws), ws.numel(),
                                    _stream(canvas)), "dq_qgemm_rows_sample")
    return token, stats, ws


def debug_subdots(type_: int, act: Act, packed: torch.Tensor, N: int) -> torch.Tensor:
    """Per-sub-block int32 dots from the GEMM kernel's own path: [M, N, K/256, J],
    J = 8 (Q4_K) or 16 (Q6_K)."""
    lib = load_library()
    M, K = _check_operands(type_, act, packed, N)
    J = 8 if type_ == Q4_K else 16
    dots = torch.empty((M, N, K // 256, J), dtype=torch.int32, device=act.buf.device)
    _check(lib.dq_debug_subdots(type_, M, N, K, _ptr(act.buf), _ptr(packed), _ptr(dots),
                                _stream(act.buf)), "dq_debug_subdots")
    return dots


def debug_superblock_sums(type_: int, act: Act, packed: torch.Tensor, N: int):
    """Exact per-(m, n, super-block) integers (S, Mn) from the GEMM kernel's own path."""
    lib = load_library()
    M, K = _check_operands(type_, act, packed, N)
    nb = K // QK
    dev = act.buf.device
    S = torch.empty((M, N, nb), dtype=torch.int32, device=dev)
    Mn = torch.empty((M, N, nb), dtype=torch.int32, device=dev)
    _check(lib.dq_debug_superblock_sums(type_, M, N, K, _ptr(act.buf), _ptr(packed), _ptr(S),
                                        _ptr(Mn), _stream(act.buf)),
           "dq_debug_superblock_sums")
    return S, Mn


ROPE_NONE, ROPE_NORM, ROPE_NEOX = 0, 1, 2


def attention_workspace(L: int, H: int, Hkv: int, D: int = 128) -> int:
    lib = load_library()
    out = ctypes.c_size_t()
    _check(lib.dq_attention_workspace(L, H, Hkv, D, ctypes.byref(out)), "dq_attention_workspace")
    return out.value


def attention(qkv: torch.Tensor, H: int, Hkv: int, D: int = 128, rope: torch.Tensor | None = None,
              rope_mode: int = ROPE_NONE, out: torch.Tensor | None = None,
              ws: torch.Tensor | None = None) -> torch.Tensor:
    """Bidirectional attention over the canvas: qkv f32 [L, >= (H + 2 Hkv) D] rows
    [Q | K | V]; rope f32 [L, D/2, 2] (cos, sin) for rope_mode NORM or NEOX;
    ws: uint8 workspace of attention_workspace(L, H, Hkv, D) bytes (allocated
    when None); returns out f32 [L, H D]."""
    lib = load_library()
    _need(qkv, torch.float32, "qkv")
    if qkv.dim() != 2 or qkv.stride(1) != 1:
        raise ValueError("qkv must be 2-D with unit column stride")
    L = qkv.shape[0]
    if qkv.shape[1] < (H + 2 * Hkv) * D:
        raise ValueError("qkv has fewer than (H + 2 Hkv) D columns")
    if rope_mode != ROPE_NONE:
        if rope is None:
            raise ValueError("rope table required for this rope_mode")
        _need(rope, torch.float32, "rope")
        if not rope.is_contiguous() or rope.numel() < L * D:
            raise ValueError("rope must be a contiguous f32 [L, D/2, 2] table")
    if out is None:
        out = torch.empty((L, H * D), dtype=torch.float32, device=qkv.device)
    _need(out, torch.float32, "out")
    if out.dim() != 2 or out.shape[0] != L or out.shape[1] < H * D or out.stride(1) != 1:
        raise ValueError("out must be [L, >= H D] with unit column stride")
    ws = _ws(attention_workspace(L, H, Hkv, D), ws, qkv.device)
    _check(lib.dq_attention(L, H, Hkv, D, _ptr(qkv), qkv.stride(0) if L > 1 else qkv.shape[1],
                            _ptr(rope) if rope is not None else None, rope_mode, _ptr(out),
                            out.stride(0) if L > 1 else out.shape[1], _ptr(ws), ws.numel(),
                            _stream(qkv)), "dq_attention")
    return out


F32, F16, Q8_0, Q5_K, BF16 = 0, 1, 8, 13, 30  # the decoder's other GGUF types


def row_bytes(type_: int, K: int) -> int:
    lib = load_library()
    out = ctypes.c_size_t()
    _check(lib.dq_row_bytes(type_, K, ctypes.byref(out)), "dq_row_bytes")
    return out.value


def embed_rows(type_: int, table: torch.Tensor, K: int, ids: torch.Tensor,
               out: torch.Tensor | None = None, flags: torch.Tensor | None = None):
    """Rows ids of a GGUF table (uint8, N rows of row_bytes(type, K)) decoded to
    f32: returns (out [M, K], flags int32 [M], 1 where an id is out of range)."""
    lib = load_library()
    _need(table, torch.uint8, "table")
    _need(ids, torch.int32, "ids")
    if not table.is_contiguous() or not ids.is_contiguous():
        raise ValueError("table and ids must be contiguous")
    rb = row_bytes(type_, K)
    N = table.numel() // rb
    M = ids.numel()
    dev = table.device
    if out is None:
        out = torch.empty((M, K), dtype=torch.float32, device=dev)
    if flags is None:
        flags = torch.empty(M, dtype=torch.int32, device=dev)
    _need(out, torch.float32, "out")
    _need(flags, torch.int32, "flags")
    if out.dim() != 2 or out.shape[0] != M or out.shape[1] < K or out.stride(1) != 1:
        raise ValueError("out must be [M, >= K] with unit column stride")
    _check(lib.dq_embed_rows(type_, N, K, _ptr(table), _ptr(ids), M, _ptr(out),
                             out.stride(0) if M > 1 else out.shape[1], _ptr(flags),
                             _stream(table)), "dq_embed_rows")
    return out, flags
