"""Parity of the HIP path (called through the C ABI) with the CPU oracle.

Bit-exact: int8 codes, scales and code sums of the quantizer; the repacked
layout; the per-super-block integers S and Mn of the GEMM's own code path; the
per-sub-block dots (unit-scale probes).  Floating point: every output within
1e-4 * T[m, n], T = sum_k |w^[n,k] * x^[m,k]| in f64 (the tolerance of the
method's statement), against the oracle's plain f64 definition.
"""
import numpy as np
import pytest

import oracle
import synth
from kq_fields import (encode_q4k_matrix, encode_q6k_matrix, random_q4k_fields,
                       random_q6k_fields)
from packed_layout import ROWS, TILE, read_tile
import act_layout

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

TOL = 1e-4


@pytest.fixture(scope="module")
def dq():
    import quantized_gemm_diffusion_amd as m
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    m.load_library()
    return m


DEV = "cuda:0"


def _t(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def _sync():
    torch.cuda.synchronize()


def _act(dq, xq, xd, xb):
    """Oracle-quantized activations in the library's record layout, on the GPU."""
    M, K = xq.shape
    return dq.Act(_t(act_layout.pack(xq, xd, xb)), M, K)


def _unpack(act):
    q, d, b, padding_ok = act_layout.unpack(act.buf.cpu().numpy(), act.M, act.K)
    assert padding_ok, "padding rows or record tails are not zero"
    return q, d, b


def _weights(type_, N, K, seed, full_scales=False):
    rng = np.random.default_rng(seed)
    if type_ == oracle.Q4_K:
        return synth.q4k_weights(rng, N, K)
    if full_scales:
        return synth.q6k_weights(rng, N, K, sc_lo=-128, sc_hi=127)
    return synth.q6k_weights(rng, N, K)


def _check_tol(y, yr, T, what):
    err = np.abs(np.asarray(y, np.float64) - yr)
    bad = err > TOL * T
    assert not bad.any(), f"{what}: {bad.sum()} outputs out of tolerance, worst err/T " \
                          f"{np.max(err / np.maximum(T, 1e-300)):.3g}"


# --------------------------------------------------------------------------- #
# Activation quantization: bit-exact                                          #
# --------------------------------------------------------------------------- #
@pytest.mark.parametrize("M,K,seed", [(1, 256, 0), (17, 512, 1), (160, 4096, 2), (5, 18944, 3)])
def test_quantize_bit_exact(dq, M, K, seed):
    x = synth.activations(np.random.default_rng(seed), M, K)
    x[0, :256] = 0.0  # a zero block
    if M > 1:
        x[1, 256 % K:256 % K + 3] = [254.0, 3.0, -5.0]  # halfway ties
    q, d, b = _unpack(dq.quantize_act(_t(x)))
    xq, xd, xb = oracle.quantize_act(x)
    assert np.array_equal(q, xq)
    assert np.array_equal(d.view(np.uint32), xd.view(np.uint32))
    assert np.array_equal(b, xb)


def test_quantize_strided_and_unaligned_rows(dq):
    rng = np.random.default_rng(5)
    big = synth.activations(rng, 9, 1024 + 65)
    xq, xd, xb = oracle.quantize_act(np.ascontiguousarray(big[:, 1:1025]))
    xt = _t(big)
    q, d, b = _unpack(dq.quantize_act(xt[:, 1:1025]))  # row stride 1089, off 16-byte alignment
    assert np.array_equal(q, xq) and np.array_equal(b, xb)
    assert np.array_equal(d, xd)


# --------------------------------------------------------------------------- #
# Repack: every bit lands where the layout says                              #
# --------------------------------------------------------------------------- #
@pytest.mark.parametrize("type_", [oracle.Q4_K, oracle.Q6_K])
def test_repack_layout(dq, type_):
    N, K = 38, 768  # three tiles, the last one ragged
    nb = K // 256
    W = _weights(type_, N, K, 40, full_scales=True)
    packed = dq.repack_weights(type_, N, K, _t(W.reshape(-1))).cpu().numpy()
    assert packed.size == dq.packed_size(type_, N, K)
    tb = TILE[type_]
    tiles = packed.reshape(-1, nb, tb)
    for nt in range(tiles.shape[0]):
        for b in range(nb):
            got = read_tile(type_, tiles[nt, b])
            for r in range(ROWS):
                n = ROWS * nt + r
                if type_ == oracle.Q4_K:
                    heads, q = got
                    if n >= N:
                        assert not heads[r].any() and not q[r].any()
                        continue
                    _, _, _, _, oq = oracle.decode_q4k(W[n, b])
                    assert np.array_equal(heads[r], W[n, b, :16])
                    assert np.array_equal(q[r], oq)
                else:
                    d_bits, sc, q = got
                    if n >= N:
                        assert d_bits[r] == 0 and not sc[r].any() and not q[r].any()
                        continue
                    _, osc, oq = oracle.decode_q6k(W[n, b])
                    assert int(d_bits[r]) == int(W[n, b, 208]) | (int(W[n, b, 209]) << 8)
                    assert np.array_equal(sc[r], osc) and np.array_equal(q[r], oq)


# --------------------------------------------------------------------------- #
# Integer part of the GEMM: bit-exact                                         #
# --------------------------------------------------------------------------- #
@pytest.mark.parametrize("type_,M,N,K", [(oracle.Q4_K, 37, 70, 768), (oracle.Q6_K, 37, 70, 768),
                                         (oracle.Q4_K, 64, 32, 256), (oracle.Q6_K, 1, 33, 512)])
def test_superblock_sums_bit_exact(dq, type_, M, N, K):
    W = _weights(type_, N, K, 50 + M, full_scales=True)
    x = synth.activations(np.random.default_rng(60 + M), M, K)
    xq, xd, xb = oracle.quantize_act(x)
    packed = dq.repack_weights(type_, N, K, _t(W.reshape(-1)))
    S, Mn = dq.debug_superblock_sums(type_, _act(dq, xq, xd, xb), packed, N)
    _sync()
    oS, oMn = oracle.superblock_sums(type_, xq, xb, W, N)
    assert np.array_equal(S.cpu().numpy(), oS)
    assert np.array_equal(Mn.cpu().numpy(), oMn)


@pytest.mark.parametrize("type_", [oracle.Q4_K, oracle.Q6_K])
def test_subblock_dots_bit_exact(dq, type_):
    # all scales 0 except sub-block j's, set to 1: S of super-block b is dot_j
    M, N, nb = 33, 40, 2
    K = 256 * nb
    rng = np.random.default_rng(70)
    x = synth.activations(rng, M, K)
    xq, xd, xb = oracle.quantize_act(x)
    J = 8 if type_ == oracle.Q4_K else 16
    f = random_q4k_fields(rng, N, nb) if type_ == oracle.Q4_K else random_q6k_fields(rng, N, nb)
    W0 = encode_q4k_matrix(f) if type_ == oracle.Q4_K else encode_q6k_matrix(f)
    dots = oracle.subdots(type_, xq, W0, N)  # [M, N, nb, J]
    for j in range(J):
        fj = dict(f)
        fj["sc"] = np.zeros_like(f["sc"])
        fj["sc"][..., j] = 1
        Wj = encode_q4k_matrix(fj) if type_ == oracle.Q4_K else encode_q6k_matrix(fj)
        packed = dq.repack_weights(type_, N, K, _t(Wj.reshape(-1)))
        S, _ = dq.debug_superblock_sums(type_, _act(dq, xq, xd, xb), packed, N)
        _sync()
        assert np.array_equal(S.cpu().numpy(), dots[..., j]), f"sub-block {j}"


@pytest.mark.parametrize("type_,M,N,K", [(oracle.Q4_K, 33, 40, 512), (oracle.Q6_K, 37, 70, 768),
                                         (oracle.Q4_K, 160, 100, 1024), (oracle.Q6_K, 20, 48, 512),
                                         (oracle.Q4_K, 512, 64, 512)])
def test_subdots_hook_bit_exact(dq, type_, M, N, K):
    # dq_debug_subdots: every per-sub-block int32 dot from the GEMM kernel's own
    # unpack + MFMA path (scales replaced by one-hot selectors), full int8 Q6_K
    # scales in the weights (the hook ignores them)
    W = _weights(type_, N, K, 300 + M + N, full_scales=True)
    x = synth.activations(np.random.default_rng(310 + M), M, K)
    xq, xd, xb = oracle.quantize_act(x)
    packed = dq.repack_weights(type_, N, K, _t(W.reshape(-1)))
    dots = dq.debug_subdots(type_, _act(dq, xq, xd, xb), packed, N)
    _sync()
    assert np.array_equal(dots.cpu().numpy(), oracle.subdots(type_, xq, W, N))


# --------------------------------------------------------------------------- #
# GEMM outputs within tolerance, tails and degenerate shapes                  #
# --------------------------------------------------------------------------- #
@pytest.mark.parametrize("type_", [oracle.Q4_K, oracle.Q6_K])
@pytest.mark.parametrize("M,N,K", [(1, 32, 256), (8, 100, 1024), (17, 33, 512), (160, 96, 768),
                                   (511, 40, 512), (16, 256, 512)])
def test_qgemm_within_tolerance(dq, type_, M, N, K):
    W = _weights(type_, N, K, 80 + M + N)
    x = synth.activations(np.random.default_rng(90 + M), M, K)
    xq, xd, xb = oracle.quantize_act(x)
    packed = dq.repack_weights(type_, N, K, _t(W.reshape(-1)))
    y = dq.qgemm(type_, _act(dq, xq, xd, xb), packed, N)
    _sync()
    yr, T = oracle.qgemm_ref(type_, xq, xd, W, N)
    _check_tol(y.cpu().numpy(), yr, T, f"type {type_} {M}x{N}x{K}")


def test_qgemm_strided_output_untouched_padding(dq):
    M, N, K = 40, 70, 512
    W = _weights(oracle.Q4_K, N, K, 3)
    xq, xd, xb = oracle.quantize_act(synth.activations(np.random.default_rng(4), M, K))
    packed = dq.repack_weights(oracle.Q4_K, N, K, _t(W.reshape(-1)))
    ybig = torch.full((M, N + 9), -7.0, device=DEV)
    dq.qgemm(oracle.Q4_K, _act(dq, xq, xd, xb), packed, N, y=ybig)
    _sync()
    yb = ybig.cpu().numpy()
    assert np.all(yb[:, N:] == -7.0)
    yr, T = oracle.qgemm_ref(oracle.Q4_K, xq, xd, W, N)
    _check_tol(yb[:, :N], yr, T, "strided y")


def test_qgemm_deterministic_and_power_of_two_scaling(dq):
    M, N, K = 160, 64, 1024
    W = _weights(oracle.Q6_K, N, K, 5)
    x = synth.activations(np.random.default_rng(6), M, K)
    packed = dq.repack_weights(oracle.Q6_K, N, K, _t(W.reshape(-1)))
    a = dq.quantize_act(_t(x))
    y1 = dq.qgemm(oracle.Q6_K, a, packed, N).cpu().numpy()
    y2 = dq.qgemm(oracle.Q6_K, a, packed, N).cpu().numpy()
    assert np.array_equal(y1.view(np.uint32), y2.view(np.uint32))
    a3 = dq.quantize_act(_t(x * np.float32(2.0 ** -5)))
    y3 = dq.qgemm(oracle.Q6_K, a3, packed, N).cpu().numpy()
    assert np.array_equal(y3, y1 * np.float32(2.0 ** -5))


def test_zero_activations_give_zero(dq):
    M, N, K = 20, 64, 512
    W = _weights(oracle.Q4_K, N, K, 8)
    packed = dq.repack_weights(oracle.Q4_K, N, K, _t(W.reshape(-1)))
    a = dq.quantize_act(torch.zeros((M, K), device=DEV))
    y = dq.qgemm(oracle.Q4_K, a, packed, N).cpu().numpy()
    assert np.all(y == 0.0)


# --------------------------------------------------------------------------- #
# Gathered-row projection                                                     #
# --------------------------------------------------------------------------- #
def test_rows_gather_matches_quantized_gemm(dq):
    L, K, N = 160, 1024, 200
    W = _weights(oracle.Q6_K, N, K, 9)
    canvas = synth.activations(np.random.default_rng(10), L, K)
    packed = dq.repack_weights(oracle.Q6_K, N, K, _t(W.reshape(-1)))
    idx = np.array([159, 0, 7, 7, 42, 3], np.int32)  # unsorted, with a duplicate
    y, ws = dq.qgemm_rows(oracle.Q6_K, _t(canvas), _t(idx), packed, N)
    _sync()
    gq, gd, gb = oracle.qgemm_rows_inputs(canvas, idx)
    yr, T = oracle.qgemm_ref(oracle.Q6_K, gq, gd, W, N)
    yn = y.cpu().numpy()
    _check_tol(yn, yr, T, "rows")
    assert np.array_equal(yn[2], yn[3])  # duplicate index, identical row
    assert not ws[: 4 * len(idx)].view(torch.int32).cpu().numpy().any()
    # gather-then-quantize equals quantize-then-gather, bit for bit
    yall = dq.qgemm(oracle.Q6_K, dq.quantize_act(_t(canvas)), packed, N).cpu().numpy()
    assert np.array_equal(yn.view(np.uint32), yall[idx].view(np.uint32))
    # permuting idx permutes the rows
    perm = np.array([3, 5, 0, 1, 2, 4])
    yp, _ = dq.qgemm_rows(oracle.Q6_K, _t(canvas), _t(idx[perm]), packed, N)
    assert np.array_equal(yp.cpu().numpy(), yn[perm])


def test_rows_out_of_range_index_is_flagged_not_read(dq):
    L, K, N = 10, 512, 64
    W = _weights(oracle.Q4_K, N, K, 11)
    canvas = synth.activations(np.random.default_rng(12), L, K)
    packed = dq.repack_weights(oracle.Q4_K, N, K, _t(W.reshape(-1)))
    idx = np.array([2, 10, -1, 9], np.int32)
    y, ws = dq.qgemm_rows(oracle.Q4_K, _t(canvas), _t(idx), packed, N)
    _sync()
    flags = ws[:16].view(torch.int32).cpu().numpy()
    assert list(flags) == [0, 1, 1, 0]
    yn = y.cpu().numpy()
    assert np.all(yn[1] == 0) and np.all(yn[2] == 0)
    gq, gd, _ = oracle.qgemm_rows_inputs(canvas, idx[[0, 3]])
    yr, T = oracle.qgemm_ref(oracle.Q4_K, gq, gd, W, N)
    _check_tol(yn[[0, 3]], yr, T, "valid rows")


@pytest.mark.parametrize("ldc_pad", [0, 1])  # 16-byte-aligned rows, and rows that are not
def test_rows_single_row_gathers_in_the_gemm(dq, ldc_pad):
    # one Q6_K row over a wide vocabulary: the gather and quantization run inside
    # the GEMM launch; codes and sums must be those of the separate quantizer, so
    # the row equals, bit for bit, the single-row GEMM of that row quantized apart
    L, K, N = 40, 2048, 20000
    W = _weights(oracle.Q6_K, N, K, 13, full_scales=True)
    canvas = np.zeros((L, K + ldc_pad), np.float32)
    canvas[:, :K] = synth.activations(np.random.default_rng(14), L, K)
    canvas[5, :256] = 0.0  # a zero block
    packed = dq.repack_weights(oracle.Q6_K, N, K, _t(W.reshape(-1)))
    ct = _t(canvas)[:, :K] if ldc_pad else _t(canvas)
    for r in (5, 0, L - 1):
        y, ws = dq.qgemm_rows(oracle.Q6_K, ct, _t(np.array([r], np.int32)), packed, N)
        y1 = dq.qgemm(oracle.Q6_K, dq.quantize_act(ct[r:r + 1]), packed, N)
        _sync()
        assert ws[:4].view(torch.int32).cpu().numpy()[0] == 0
        yn = y.cpu().numpy()[0]
        assert np.array_equal(yn.view(np.uint32), y1.cpu().numpy()[0].view(np.uint32)), r
        gq, gd, _ = oracle.qgemm_rows_inputs(canvas[:, :K], np.array([r], np.int32))
        yr, T = oracle.qgemm_ref(oracle.Q6_K, gq, gd, W, N)
        _check_tol(yn[None, :], yr, T, f"single row {r}")
    for bad in (L, -3):
        y, ws = dq.qgemm_rows(oracle.Q6_K, ct, _t(np.array([bad], np.int32)), packed, N)
        _sync()
        assert ws[:4].view(torch.int32).cpu().numpy()[0] == 1
        assert np.all(y.cpu().numpy() == 0)


# --------------------------------------------------------------------------- #
# ABI errors through the binding on the GPU                                   #
# --------------------------------------------------------------------------- #
def test_abi_errors_on_gpu(dq):
    act = dq.quantize_act(torch.zeros((4, 512), device=DEV))
    packed = torch.zeros(dq.packed_size(dq.Q4_K, 32, 512), dtype=torch.uint8, device=DEV)
    with pytest.raises(ValueError):
        dq.qgemm(dq.Q4_K, act, packed[:-1], 32)  # packed too small
    with pytest.raises(ValueError):
        dq.qgemm(dq.Q4_K, dq.Act(act.buf[:-16], 4, 512), packed, 32)  # activations too small
    lib = dq.load_library()
    y = torch.zeros((4, 32), device=DEV)
    sp = torch.cuda.current_stream().cuda_stream
    assert lib.dq_qgemm(dq.Q4_K, 4, 32, 500, act.buf.data_ptr(), packed.data_ptr(),
                        y.data_ptr(), 32, sp) == dq.DQ_EINVAL  # K not a multiple of 256
    assert lib.dq_qgemm(dq.Q4_K, 4, 32, 512, act.buf.data_ptr() + 4, packed.data_ptr(),
                        y.data_ptr(), 32, sp) == dq.DQ_EINVAL  # misaligned activations
    assert lib.dq_qgemm(7, 4, 32, 512, act.buf.data_ptr(), packed.data_ptr(),
                        y.data_ptr(), 32, sp) == dq.DQ_EUNSUPPORTED
    canvas = torch.zeros((8, 512), device=DEV)
    idx = torch.zeros(4, dtype=torch.int32, device=DEV)
    with pytest.raises(dq.DQError) as e:
        dq.qgemm_rows(dq.Q4_K, canvas, idx, packed, 32,
                      ws=torch.zeros(16, dtype=torch.uint8, device=DEV))
    assert e.value.status == dq.DQ_EWORKSPACE


# --------------------------------------------------------------------------- #
# m-tilings of the GEMM (the launcher picks the 16-row blocks per workgroup   #
# from M and N): shapes chosen so that several choices are exercised          #
# --------------------------------------------------------------------------- #
@pytest.mark.parametrize("type_,M,N,K", [
    (oracle.Q4_K, 160, 8192, 512),    # 10 blocks of 16 rows in 2 workgroup rows
    (oracle.Q6_K, 128, 8200, 512),    # ragged N
    (oracle.Q4_K, 96, 8192, 1280),    # 5 super-blocks over 4 waves
    (oracle.Q6_K, 64, 8192, 256),     # a single super-block
    (oracle.Q4_K, 150, 8224, 768),    # a ragged last 16-row block
    (oracle.Q4_K, 160, 12270, 512),   # three n-tiles per wave, ragged last column group
    (oracle.Q4_K, 160, 4096, 4096),   # 8 waves over 16 super-blocks
    (oracle.Q6_K, 64, 24568, 512),    # Q6_K, three n-tiles per wave, ragged last n-tile
    (oracle.Q4_K, 160, 24560, 512),   # three n-tiles, 2-wave workgroups (1024 of them)
    (oracle.Q6_K, 64, 49144, 512),    # Q6_K, three n-tiles, 2-wave workgroups
    (oracle.Q4_K, 512, 8192, 768),    # 8 m-blocks, 2-wave workgroups, 3 super-blocks over 2 waves
])
def test_qgemm_every_m_tiling(dq, type_, M, N, K):
    W = _weights(type_, N, K, 300 + M, full_scales=True)
    x = synth.activations(np.random.default_rng(400 + M), M, K)
    xq, xd, xb = oracle.quantize_act(x)
    packed = dq.repack_weights(type_, N, K, _t(W.reshape(-1)))
    y = dq.qgemm(type_, _act(dq, xq, xd, xb), packed, N)
    _sync()
    yr, T = oracle.qgemm_ref(type_, xq, xd, W, N)
    _check_tol(y.cpu().numpy(), yr, T, f"type {type_} {M}x{N}x{K}")


@pytest.mark.parametrize("type_,M,N", [(oracle.Q4_K, 160, 8192), (oracle.Q6_K, 128, 8192),
                                       (oracle.Q4_K, 64, 8192),
                                       (oracle.Q4_K, 160, 12270),   # three n-tiles per wave
                                       (oracle.Q6_K, 64, 24568),
                                       (oracle.Q4_K, 160, 24560),   # 2-wave workgroups
                                       (oracle.Q4_K, 512, 8192)])
def test_superblock_sums_bit_exact_multi_tile(dq, type_, M, N):
    K = 512
    W = _weights(type_, N, K, 500 + M, full_scales=True)
    x = synth.activations(np.random.default_rng(600 + M), M, K)
    xq, xd, xb = oracle.quantize_act(x)
    packed = dq.repack_weights(type_, N, K, _t(W.reshape(-1)))
    S, Mn = dq.debug_superblock_sums(type_, _act(dq, xq, xd, xb), packed, N)
    _sync()
    oS, oMn = oracle.superblock_sums(type_, xq, xb, W, N)
    assert np.array_equal(S.cpu().numpy(), oS)
    assert np.array_equal(Mn.cpu().numpy(), oMn)


# --------------------------------------------------------------------------- #
# Narrow M (at most 32 rows, K of 8 to 16 super-blocks, at least 1,024        #
# n-tiles): the persistent weight-streaming kernel.  Every output is compared #
# with the oracle; padding columns of a strided output stay untouched.        #
# --------------------------------------------------------------------------- #
@pytest.mark.parametrize("type_,M,N,K,pad", [
    (oracle.Q6_K, 32, 16400, 4096, 0),   # two 16-row blocks, 8 waves, ragged last n-tile
    (oracle.Q4_K, 17, 16390, 2048, 0),   # ragged rows, N % 4 != 0 (element stores), 4 waves
    (oracle.Q6_K, 1, 20000, 3584, 0),    # one row, 7 waves
    (oracle.Q4_K, 32, 16384, 4096, 3),   # row stride N + 3 (element stores)
    (oracle.Q6_K, 16, 32776, 2560, 0),   # 5 waves, many n-tiles per workgroup
    (oracle.Q4_K, 5, 16384, 4096, 0),    # one partial 16-row block, vector stores
    (oracle.Q6_K, 1, 16390, 4096, 0),    # one row (sub-blocks as operand rows), element stores
    (oracle.Q6_K, 1, 32768, 2560, 2),    # one row, 5 waves, vector stores
    (oracle.Q6_K, 2, 16400, 4096, 0),    # 2 to 4 rows: k-quarters as operand rows
    (oracle.Q6_K, 3, 16390, 2048, 3),    # 3 rows, row stride N + 3, ragged n-tile
    (oracle.Q6_K, 4, 20000, 3584, 0),    # 4 rows, 7 waves
    (oracle.Q6_K, 5, 16390, 2048, 3),    # 5 rows: back on the narrow kernel
])
def test_qgemm_narrow_m(dq, type_, M, N, K, pad):
    W = _weights(type_, N, K, 700 + M + K // 256, full_scales=True)
    x = synth.activations(np.random.default_rng(800 + M), M, K)
    xq, xd, xb = oracle.quantize_act(x)
    packed = dq.repack_weights(type_, N, K, _t(W.reshape(-1)))
    ybig = torch.full((M, N + pad), -7.0, device=DEV)
    dq.qgemm(type_, _act(dq, xq, xd, xb), packed, N, y=ybig)
    _sync()
    yb = ybig.cpu().numpy()
    assert np.all(yb[:, N:] == -7.0)
    yr, T = oracle.qgemm_ref(type_, xq, xd, W, N)
    _check_tol(yb[:, :N], yr, T, f"narrow type {type_} {M}x{N}x{K}")
