"""Parity of the shared-record canvas kernel (one n-tile per wave, activation
records shared by the waves of a K-part, two K-parts per workgroup).

The launcher takes it where its grid is one round of workgroups that fills
at least 70% of the CUs; on MI355X (256 CUs) every shape below does (160, 128
and 80-row variants, Q4_K and Q6_K), with ragged M and N, K-parts of unequal
length (odd super-block counts), a strided output, and signed, zero and
subnormal super-block scales.  Outputs within 1e-4 * T of the oracle's f64
plain definition; per-super-block S and Mn bit-exact through the debug mode,
which runs the same kernel.
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


def _weights(type_, N, K, seed, mixed=False):
    rng = np.random.default_rng(seed)
    if type_ == oracle.Q4_K:
        return synth.q4k_weights(rng, N, K, mixed_scales=mixed)
    return synth.q6k_weights(rng, N, K, sc_lo=-128, sc_hi=127, mixed_scales=mixed)


def _act(dq, xq, xd, xb):
    M, K = xq.shape
    return dq.Act(_t(act_layout.pack(xq, xd, xb)), M, K)


# (type, M, N, K, row-stride padding, mixed scales): 160-row variant at 150 and
# 160 rows, 128-row variant at 250 rows (two row groups), 80-row variant at 75
# and 80 rows; 5, 6, 7, 9 and 4 super-blocks
CASES = [
    (oracle.Q4_K, 150, 20000, 1280, 0, False),
    (oracle.Q6_K, 160, 19000, 1536, 0, True),
    (oracle.Q4_K, 250, 11190, 1792, 0, False),
    (oracle.Q4_K, 75, 18000, 2304, 0, True),
    (oracle.Q6_K, 80, 17700, 1024, 3, False),
]


@pytest.mark.parametrize("type_,M,N,K,pad,mixed", CASES)
def test_shared_record_kernel_within_tolerance(dq, type_, M, N, K, pad, mixed):
    print(f"shared-record GEMM type {type_} {M}x{N}x{K} pad {pad}", flush=True)
    W = _weights(type_, N, K, M + N + K, mixed)
    x = synth.activations(np.random.default_rng(M * 3 + K), M, K)
    xq, xd, xb = oracle.quantize_act(x)
    packed = dq.repack_weights(type_, N, K, _t(W.reshape(-1)))
    ybig = torch.full((M, N + pad), -7.0, device=DEV)
    dq.qgemm(type_, _act(dq, xq, xd, xb), packed, N, y=ybig)
    torch.cuda.synchronize()
    yb = ybig.cpu().numpy()
    if pad:
        assert np.all(yb[:, N:] == -7.0), "stores past column N"
    yy = yb[:, :N].astype(np.float64)
    assert np.all(np.isfinite(yy))
    yr, T = oracle.qgemm_ref(type_, xq, xd, W, N)
    err = np.abs(yy - yr)
    bad = err > TOL * T
    assert not bad.any(), f"{bad.sum()} outputs out of tolerance, worst err/T " \
                          f"{np.max(err / np.maximum(T, 1e-300)):.3g}"


@pytest.mark.parametrize("type_,M,N,K", [(oracle.Q4_K, 145, 17200, 1024),
                                         (oracle.Q6_K, 80, 17700, 1024)])
def test_shared_record_superblock_sums_bit_exact(dq, type_, M, N, K):
    print(f"shared-record sums type {type_} {M}x{N}x{K}", flush=True)
    W = _weights(type_, N, K, 7 * M + N)
    x = synth.activations(np.random.default_rng(11 * M), M, K)
    xq, xd, xb = oracle.quantize_act(x)
    packed = dq.repack_weights(type_, N, K, _t(W.reshape(-1)))
    S, Mn = dq.debug_superblock_sums(type_, _act(dq, xq, xd, xb), packed, N)
    torch.cuda.synchronize()
    oS, oMn = oracle.superblock_sums(type_, xq, xb, W, N)
    assert np.array_equal(S.cpu().numpy(), oS)
    assert np.array_equal(Mn.cpu().numpy(), oMn)


@pytest.mark.parametrize("type_,M,N,K", [(oracle.Q4_K, 145, 17200, 1024),
                                         (oracle.Q6_K, 80, 17700, 1024)])
def test_shared_record_subdots_bit_exact(dq, type_, M, N, K):
    # every per-sub-block int32 dot through the shared-record kernel's own path
    print(f"shared-record sub-block dots type {type_} {M}x{N}x{K}", flush=True)
    W = _weights(type_, N, K, 13 * M + N)
    x = synth.activations(np.random.default_rng(17 * M), M, K)
    xq, xd, xb = oracle.quantize_act(x)
    packed = dq.repack_weights(type_, N, K, _t(W.reshape(-1)))
    dots = dq.debug_subdots(type_, _act(dq, xq, xd, xb), packed, N)
    torch.cuda.synchronize()
    assert np.array_equal(dots.cpu().numpy(), oracle.subdots(type_, xq, W, N))
