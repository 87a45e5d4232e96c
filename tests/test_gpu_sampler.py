"""Sampler statistics of requested logits rows on the GPU (through the C ABI).

dq_logits_stats on seeded f32 logits against the oracle on the same values:
the token (first maximum of the binary32 product beta * y) and the maximum
bit for bit, the log-partition, entropy and top probability within binary32
summation error.

dq_qgemm_rows_sample (the statistics formed in the projection's epilogue):
  * against the oracle's plain f64 logits of the same rows, at sizes the
    oracle finishes in seconds, on both GEMM kernels (the canvas kernel and
    the narrow one that serves at most 32 rows): every statistic within the
    bounds that follow from the GEMM tolerance |y - y_ref| <= 1e-4 * T (with
    e = beta * 1e-4 * max_n T[row, n]: max within e, the token's oracle value
    within 2e of the oracle maximum, log-partition within e, entropy within
    e * exp(2e) * (D + 2e) where D = sum_n p[n] |z[n] - mean_p z|, top
    probability within a factor exp(2e)), plus the binary32 summation error;
  * at the output projection's real shapes (126,464 x 4096 on 1, 8, 32 rows;
    152,064 x 3584 on 64 rows), against the logits dq_qgemm_rows writes for
    the same arguments (the two share the GEMM's accumulation, so the token
    and maximum must agree bit for bit), and on sampled rows against the
    oracle's f64 logits within the bounds above;
  * an index outside [0, L) at one row (the in-GEMM gather): flagged, the row
    taken as zeros, so its statistics are those of N equal logits;
  * edge cases: a single row, duplicate and unsorted indices, ties at the
    maximum (the first column wins), flat and peaked temperatures.
"""
import numpy as np
import pytest

import oracle
import synth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

DEV = "cuda:0"
TOL = 1e-4          # GEMM output tolerance, relative to T
SUM_TOL = 3e-5      # binary32 sums of exponentials (relative)


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
    return synth.q4k_weights(rng, N, K) if type_ == oracle.Q4_K else synth.q6k_weights(rng, N, K)


def _check_exact_inputs(tok, st, tok_r, st_r, what):
    """GPU statistics of the same binary32 logits as the oracle's."""
    np.testing.assert_array_equal(tok, tok_r, err_msg=f"{what}: token")
    np.testing.assert_array_equal(st[:, 0], st_r[:, 0].astype(np.float32), err_msg=f"{what}: max")
    lse_tol = SUM_TOL * (1.0 + np.abs(st_r[:, 1] - st_r[:, 0]))
    assert np.all(np.abs(st[:, 1] - st_r[:, 1]) <= lse_tol + 1e-7 * np.abs(st_r[:, 1])), what
    assert np.all(np.abs(st[:, 2] - st_r[:, 2]) <= SUM_TOL * (1.0 + st_r[:, 2])), what
    np.testing.assert_allclose(st[:, 3], st_r[:, 3], rtol=SUM_TOL, err_msg=f"{what}: top p")


def _run_stats(dq, y, beta):
    tok, st, _ = dq.logits_stats(y, beta)
    torch.cuda.synchronize()
    return tok.cpu().numpy(), st.cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("M,N,scale,beta,seed", [
    (1, 1, 1.0, 1.0, 0),              # one column
    (3, 4097, 3.0, 1.0, 1),           # ragged tail of a chunk and of a group of 4
    (5, 126464, 64.0, 1.0 / 64, 2),   # vocabulary width, softened
    (4, 152064, 64.0, 1.0, 3),        # peaked (top probability near 1)
    (2, 50000, 1.0, 1e-3, 4),         # nearly flat (entropy near log N)
])
def test_logits_stats_matches_oracle(dq, M, N, scale, beta, seed):
    y = (np.random.default_rng(seed).standard_normal((M, N)) * scale).astype(np.float32)
    tok, st = _run_stats(dq, _t(y), beta)
    tok_r, st_r = oracle.logits_stats(y.astype(np.float64), beta)
    _check_exact_inputs(tok, st, tok_r, st_r, f"{M}x{N}")


def test_logits_stats_strided_rows_ties_and_unaligned(dq):
    rng = np.random.default_rng(7)
    M, N, ld = 6, 9001, 9003
    buf = (rng.standard_normal((M, ld)) * 5).astype(np.float32)
    # ties at the maximum: the first column must win
    buf[1, [17, 4000, 9000]] = 100.0
    buf[2, [8999, 9000]] = 100.0
    buf[3, :N] = 0.25                      # all equal
    y = _t(buf)[:, :N]                     # row stride 9003 floats: the scalar load path
    tok, st = _run_stats(dq, y, 0.5)
    tok_r, st_r = oracle.logits_stats(buf[:, :N].astype(np.float64), 0.5)
    _check_exact_inputs(tok, st, tok_r, st_r, "strided")
    assert tok[1] == 17 and tok[2] == 8999 and tok[3] == 0


def _oracle_bounds(y_ref, T, beta):
    """Per-row bounds on the statistics of logits within 1e-4 * T of y_ref."""
    z = beta * y_ref
    e = beta * TOL * T.max(axis=1)
    zmax = z.max(axis=1)
    p = np.exp(z - zmax[:, None])
    p /= p.sum(axis=1, keepdims=True)
    zbar = (p * z).sum(axis=1)
    D = (p * np.abs(z - zbar[:, None])).sum(axis=1)
    return z, e, e * np.exp(2 * e) * (D + 2 * e)


def _check_against_reference(tok, st, y_ref, T, beta, what):
    tok_r, st_r = oracle.logits_stats(y_ref, beta)
    z, e, dh = _oracle_bounds(y_ref, T, beta)
    rows = np.arange(len(tok))
    f32 = 2.0 ** -23 * np.abs(st_r[:, 0])  # the binary32 rounding of the product itself
    assert np.all(np.abs(st[:, 0] - st_r[:, 0]) <= e + 2 * f32), f"{what}: max"
    assert np.all(z[rows, tok] >= st_r[:, 0] - 2 * e - 2 * f32), f"{what}: token not a maximum"
    lse_sum = SUM_TOL * (1 + st_r[:, 1] - st_r[:, 0])
    assert np.all(np.abs(st[:, 1] - st_r[:, 1]) <= e + 2 * f32 + lse_sum), f"{what}: log-partition"
    assert np.all(np.abs(st[:, 2] - st_r[:, 2]) <= dh + 2 * f32 + SUM_TOL * (1 + st_r[:, 2])), \
        f"{what}: entropy"
    ratio = st[:, 3] / st_r[:, 3]
    assert np.all(np.abs(np.log(ratio)) <= 2 * e + 4 * f32 + SUM_TOL), f"{what}: top probability"
    # where the oracle's top two are further apart than the error, the token is unique
    zs = np.sort(z, axis=1)
    clear = zs[:, -1] - zs[:, -2] > 2 * e + 4 * f32
    assert np.array_equal(tok[clear], tok_r[clear]), f"{what}: token"


@pytest.mark.parametrize("type_,L,M,N,K,beta", [
    (oracle.Q6_K, 40, 20, 3000, 512, 0.05),    # canvas kernel, ragged N and M
    (oracle.Q4_K, 37, 17, 1000, 768, 0.1),     # canvas kernel, Q4_K
    (oracle.Q6_K, 160, 32, 16400, 2048, 0.02),  # narrow kernel, 2 blocks of 16 rows
    (oracle.Q6_K, 160, 1, 16390, 2048, 1.0),   # narrow kernel, one row, ragged N
    (oracle.Q6_K, 64, 4, 16390, 2048, 0.3),    # 2 to 4 rows, a duplicate
    (oracle.Q4_K, 64, 9, 16384, 2560, 0.05),   # narrow kernel, Q4_K, 5 waves
])
def test_rows_sample_against_oracle(dq, type_, L, M, N, K, beta):
    rng = np.random.default_rng(1000 + M)
    W = _weights(type_, N, K, 2000 + N)
    canvas = synth.activations(rng, L, K)
    idx = rng.permutation(L)[:M].astype(np.int32)
    if M > 2:
        idx[1] = idx[0]  # a duplicate
    packed = dq.repack_weights(type_, N, K, _t(W.reshape(-1)))
    tok, st, ws = dq.qgemm_rows_sample(type_, _t(canvas), _t(idx), packed, N, beta)
    torch.cuda.synchronize()
    tok, st = tok.cpu().numpy(), st.cpu().numpy().astype(np.float64)
    assert not ws[: 4 * M].view(torch.int32).cpu().numpy().any()
    _, _, y_ref, T = oracle.qgemm_rows_sample_ref(type_, canvas, idx, W, N, beta)
    _check_against_reference(tok, st, y_ref, T, beta, f"{type_} {M}x{N}x{K}")
    if M > 2:
        assert tok[0] == tok[1] and np.array_equal(st[0], st[1])


@pytest.mark.parametrize("type_,L,M,N,K,beta", [
    (oracle.Q6_K, 160, 32, 126464, 4096, 1.0 / 64),  # LLaDA output projection, 32 rows
    (oracle.Q6_K, 160, 8, 126464, 4096, 1.0),
    (oracle.Q6_K, 160, 1, 126464, 4096, 0.01),
    (oracle.Q6_K, 160, 3, 126464, 4096, 0.5),        # 2 to 4 rows
    (oracle.Q6_K, 512, 64, 152064, 3584, 1.0 / 64),  # Dream output projection, 64 rows
])
def test_rows_sample_matches_rows_logits_at_full_size(dq, type_, L, M, N, K, beta):
    rng = np.random.default_rng(synth.seed(4, 0, M))
    W = synth.q6k_weights(rng, N, K)
    canvas = synth.activations(rng, L, K)
    idx = synth.row_index(rng, L, M)
    packed = dq.repack_weights(type_, N, K, _t(W.reshape(-1)))
    c, i = _t(canvas), _t(idx)
    y, _ = dq.qgemm_rows(type_, c, i, packed, N)
    tok, st, _ = dq.qgemm_rows_sample(type_, c, i, packed, N, beta)
    torch.cuda.synchronize()
    yb = np.float32(beta) * y.cpu().numpy()  # the same binary32 product
    tok, st = tok.cpu().numpy(), st.cpu().numpy().astype(np.float64)
    tok_r, st_r = oracle.logits_stats(yb.astype(np.float64), 1.0)
    _check_exact_inputs(tok, st, tok_r, st_r, f"{M}x{N}x{K}")
    # and against the oracle's own f64 logits of sampled rows (first, last, one more)
    rows = np.unique([0, M - 1, int(rng.integers(0, M))])
    gq, gd, _ = oracle.qgemm_rows_inputs(canvas, idx[rows])
    y_ref, T = oracle.qgemm_ref(type_, gq, gd, W, N)
    _check_against_reference(tok[rows], st[rows], y_ref, T, beta, f"{M}x{N}x{K} rows {rows}")


def test_rows_sample_tie_goes_to_first_column(dq):
    type_, L, M, N, K = oracle.Q6_K, 48, 4, 16400, 2048
    rng = np.random.default_rng(77)
    W = synth.q6k_weights(rng, N, K)
    canvas = synth.activations(rng, L, K)
    idx = np.array([5, 9, 30, 47], np.int32)
    c, i = _t(canvas), _t(idx)
    packed = dq.repack_weights(type_, N, K, _t(W.reshape(-1)))
    tok0, st0, _ = dq.qgemm_rows_sample(type_, c, i, packed, N, 1.0)
    tok0, st0 = tok0.cpu().numpy(), st0.cpu().numpy()
    t = int(tok0[0])
    # copy row 0's winning weight row to a column 5000 before or after it (another
    # tile, handled by another workgroup): the two logits are bit-identical, and
    # the smaller column must win
    for p in (t - 5000, t + 5000):
        if not 0 <= p < N:
            continue
        W2 = W.copy()
        W2[p] = W[t]
        packed2 = dq.repack_weights(type_, N, K, _t(W2.reshape(-1)))
        tok, st, _ = dq.qgemm_rows_sample(type_, c, i, packed2, N, 1.0)
        tok, st = tok.cpu().numpy(), st.cpu().numpy()
        assert tok[0] == min(p, t), (p, t, tok[0])
        assert st[0, 0] == st0[0, 0]


@pytest.mark.parametrize("bad", [160, -1])
def test_rows_sample_single_row_out_of_range_index(dq, bad):
    # one row over a wide vocabulary takes the single-row kernel, which gathers and
    # quantizes the row itself: an index outside [0, L) is flagged and the row is
    # zeros, so every logit is 0 (token 0, max 0, lse = entropy = log N, p = 1/N)
    L, K, N = 160, 4096, 126464
    W = synth.q6k_weights(np.random.default_rng(31), N, K)
    canvas = synth.activations(np.random.default_rng(32), L, K)
    packed = dq.repack_weights(oracle.Q6_K, N, K, _t(W.reshape(-1)))
    tok, st, ws = dq.qgemm_rows_sample(oracle.Q6_K, _t(canvas), _t(np.array([bad], np.int32)),
                                       packed, N, 0.7)
    torch.cuda.synchronize()
    assert ws[:4].view(torch.int32).cpu().numpy()[0] == 1
    tok, st = tok.cpu().numpy(), st.cpu().numpy().astype(np.float64)
    assert tok[0] == 0 and st[0, 0] == 0.0
    logn = np.log(N)
    assert abs(st[0, 1] - logn) <= SUM_TOL * logn and abs(st[0, 2] - logn) <= SUM_TOL * logn
    assert abs(st[0, 3] * N - 1.0) <= SUM_TOL
