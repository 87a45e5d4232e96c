"""Super-block scales of every sign and size, on every GEMM kernel.

The K-quant formats store d (and dmin) as plain fp16: a block may carry a
negative, zero (of either sign) or subnormal scale, and Q6_K sub-block scales
span the whole int8 range, so no kernel may assume a positive or normal
scale.  Each case draws d and dmin from a mixture of positive and negative
normal values, signed zeros and subnormals (synth, ``mixed_scales``) and
checks, through the C ABI:
  * every output within 1e-4 * T of the oracle's plain f64 definition;
  * the exact super-block integers S and Mn of the canvas kernel's own path;
  * scaling every d and dmin by 2**4 (exact in fp16 for these values, also for
    subnormals) scales every output by exactly 2**4, bit for bit, on the
    canvas, narrow, single-row and 2-4-row kernels.
"""
import numpy as np
import pytest

import oracle
import synth
import act_layout

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

DEV = "cuda:0"
TOL = 1e-4


@pytest.fixture(scope="module")
def dq():
    import quantized_gemm_diffusion_amd as m
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    m.load_library()
    return m


def _t(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def _weights(type_, N, K, seed):
    rng = np.random.default_rng(seed)
    if type_ == oracle.Q4_K:
        return synth.q4k_weights(rng, N, K, mixed_scales=True)
    return synth.q6k_weights(rng, N, K, sc_lo=-128, sc_hi=127, mixed_scales=True)


def _scaled_by_16(type_, W):
    """The same blocks with d (and dmin) multiplied by 16 (exact: the values
    are below 4096 in magnitude, subnormals included)."""
    W2 = W.copy()
    fields = [(0, 2), (2, 4)] if type_ == oracle.Q4_K else [(208, 210)]
    for a, b in fields:
        v = np.ascontiguousarray(W[..., a:b]).view(np.float16)
        s = (v.astype(np.float32) * np.float32(16.0)).astype(np.float16)
        assert np.array_equal(s.astype(np.float32), v.astype(np.float32) * np.float32(16.0))
        W2[..., a:b] = s.view(np.uint8)
    return W2


def _check_tol(y, yr, T, what):
    err = np.abs(np.asarray(y, np.float64) - yr)
    bad = err > TOL * T
    assert not bad.any(), f"{what}: {bad.sum()} outputs out of tolerance, worst err/T " \
                          f"{np.max(err / np.maximum(T, 1e-300)):.3g}"


SHAPES = [
    # canvas kernel, several launch shapes
    (oracle.Q4_K, 37, 70, 768),       # ragged rows and columns
    (oracle.Q6_K, 37, 70, 768),
    (oracle.Q4_K, 160, 8192, 512),    # two workgroup rows of 5 blocks
    (oracle.Q4_K, 160, 24560, 512),   # three n-tiles per wave, 2-wave workgroups
    (oracle.Q6_K, 64, 24568, 512),    # Q6_K, three n-tiles per wave
    (oracle.Q4_K, 160, 4096, 4096),   # 8 waves over 16 super-blocks
    (oracle.Q6_K, 128, 4096, 4096),
    (oracle.Q4_K, 512, 8192, 768),    # 8 m-blocks per workgroup
    # narrow kernel (at most 32 rows, wide N)
    (oracle.Q4_K, 17, 16390, 2048),
    (oracle.Q6_K, 32, 16400, 4096),
    (oracle.Q4_K, 5, 16384, 4096),
    # single-row and 2-4-row Q6_K kernels
    (oracle.Q6_K, 1, 16390, 4096),
    (oracle.Q6_K, 3, 16390, 2048),
    (oracle.Q6_K, 4, 20000, 3584),
]


@pytest.mark.parametrize("type_,M,N,K", SHAPES)
def test_mixed_sign_zero_subnormal_scales(dq, type_, M, N, K):
    W = _weights(type_, N, K, 31 * M + N + K)
    x = synth.activations(np.random.default_rng(M + 7 * N), M, K)
    xq, xd, xb = oracle.quantize_act(x)
    act = dq.Act(_t(act_layout.pack(xq, xd, xb)), M, K)
    packed = dq.repack_weights(type_, N, K, _t(W.reshape(-1)))
    y = dq.qgemm(type_, act, packed, N).cpu().numpy()
    yr, T = oracle.qgemm_ref(type_, xq, xd, W, N)
    _check_tol(y, yr, T, f"type {type_} {M}x{N}x{K}")
    # the exact integers of the canvas kernel's own path (small shapes)
    if M * N * K <= 160 * 8192 * 512:
        S, Mn = dq.debug_superblock_sums(type_, act, packed, N)
        oS, oMn = oracle.superblock_sums(type_, xq, xb, W, N)
        assert np.array_equal(S.cpu().numpy(), oS)
        assert np.array_equal(Mn.cpu().numpy(), oMn)
    # d and dmin times 16: every output times 16, bit for bit
    W16 = _scaled_by_16(type_, W)
    packed16 = dq.repack_weights(type_, N, K, _t(W16.reshape(-1)))
    y16 = dq.qgemm(type_, act, packed16, N).cpu().numpy()
    assert np.array_equal(y16, y * np.float32(16.0)), f"type {type_} {M}x{N}x{K}: 2^4 scaling"


def test_all_zero_scales_give_zero(dq):
    # d = dmin = 0 (either sign) everywhere: every dequantized weight is zero
    for type_, M, N, K in [(oracle.Q4_K, 40, 4096, 1024), (oracle.Q6_K, 1, 16390, 4096),
                           (oracle.Q6_K, 20, 16390, 2048)]:
        W = _weights(type_, N, K, 5)
        fields = [(0, 2), (2, 4)] if type_ == oracle.Q4_K else [(208, 210)]
        for a, b in fields:
            W[..., a + 1] &= 0x80  # keep the sign bit only
            W[..., a] = 0
        x = synth.activations(np.random.default_rng(6), M, K)
        act = dq.quantize_act(_t(x))
        packed = dq.repack_weights(type_, N, K, _t(W.reshape(-1)))
        y = dq.qgemm(type_, act, packed, N).cpu().numpy()
        assert np.all(y == 0.0), f"type {type_} {M}x{N}x{K}"


@pytest.mark.parametrize("M", [1, 3, 9, 40])
def test_rows_mixed_scales(dq, M):
    # the gathered-row projection (with the in-GEMM gather at one row)
    L, K, N = 160, 4096, 16400
    W = _weights(oracle.Q6_K, N, K, 900 + M)
    canvas = synth.activations(np.random.default_rng(901 + M), L, K)
    idx = synth.row_index(np.random.default_rng(902 + M), L, M)
    packed = dq.repack_weights(oracle.Q6_K, N, K, _t(W.reshape(-1)))
    y, _ = dq.qgemm_rows(oracle.Q6_K, _t(canvas), _t(idx), packed, N)
    gq, gd, _ = oracle.qgemm_rows_inputs(canvas, idx)
    yr, T = oracle.qgemm_ref(oracle.Q6_K, gq, gd, W, N)
    _check_tol(y.cpu().numpy(), yr, T, f"rows M={M}")
