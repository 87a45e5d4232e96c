"""dq_qgemm_rows_noalloc (the gathered-row projection for callers that cannot
allocate: its workspace is the library's built-in per-GPU device array)
against dq_qgemm_rows on the same arguments, through the C ABI: outputs and
index flags bit for bit, on calls in a row where each later call is smaller
than the one before (the array keeps the previous call's contents, so stale
bytes would show).  Also: sizes beyond the array are rejected with
DQ_EWORKSPACE and leave the output untouched."""
import ctypes

import numpy as np
import pytest

import oracle
import synth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module")
def dq():
    import quantized_gemm_diffusion_amd as m
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    m.load_library()
    return m


def _t(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def _call(dq, type_, canvas, idx, packed, N, y, flags):
    lib = dq.load_library()
    L, K = canvas.shape
    M = idx.numel()
    return lib.dq_qgemm_rows_noalloc(type_, L, M, N, K, canvas.data_ptr(), canvas.stride(0),
                                     idx.data_ptr(), packed.data_ptr(), y.data_ptr(), y.stride(0),
                                     None if flags is None else flags.data_ptr(),
                                     torch.cuda.current_stream().cuda_stream)


# each sequence: (type, L, K, N) and the index lists of consecutive calls, the later
# ones smaller (fewer rows)
CASES = [
    (oracle.Q6_K, 160, 4096, 16400, [[159, 0, 7, 7, 42, 3, 100, 101, 5, 6, 8, 9, 10, 11, 12, 13,
                                      14, 15, 16, 17, 18, 19, 20, 21, 22, 23, 24, 25, 26, 27, 28,
                                      29], [40, 2, 170, -1, 33]]),  # narrow kernel, then 5 rows
    (oracle.Q4_K, 200, 1024, 3000, [list(range(0, 200, 4)), [1, 3, 5, 199, 0, 7, 9, 11, 13, 15,
                                                            17, 19, 21, 23, 25, 27, 29]]),
    (oracle.Q6_K, 64, 4096, 16390, [[3, 9, 2, 60], [63]]),            # 4 rows, then one row
    (oracle.Q6_K, 64, 4096, 16390, [[5], [64]]),                       # the in-GEMM gather
]


@pytest.mark.parametrize("type_,L,K,N,calls", CASES)
@pytest.mark.parametrize("own_flags", [False, True])
def test_noalloc_matches_rows(dq, type_, L, K, N, calls, own_flags):
    W = synth.weights(np.random.default_rng(L + K + N), type_, N, K)
    canvas = _t(synth.activations(np.random.default_rng(L * 3 + 1), L, K))
    packed = dq.repack_weights(type_, N, K, _t(W.reshape(-1)))
    for ids in calls:
        idx = _t(np.array(ids, np.int32))
        M = len(ids)
        y_ref, ws = dq.qgemm_rows(type_, canvas, idx, packed, N)
        y = torch.full((M, N), -3.0, device=DEV)
        flags = torch.full((M,), 7, dtype=torch.int32, device=DEV) if own_flags else None
        assert _call(dq, type_, canvas, idx, packed, N, y, flags) == dq.DQ_OK, \
            dq.load_library().dq_last_error()
        torch.cuda.synchronize()
        assert np.array_equal(y.cpu().numpy().view(np.uint32),
                              y_ref.cpu().numpy().view(np.uint32)), (type_, M)
        if own_flags:
            want = ws[: 4 * M].view(torch.int32).cpu().numpy()
            assert np.array_equal(flags.cpu().numpy(), want)
            assert np.array_equal(want, ((np.array(ids) < 0) | (np.array(ids) >= L)).astype(
                np.int32))


def test_noalloc_rejects_sizes_beyond_the_array(dq):
    type_, L, K, N = oracle.Q4_K, 300, 16384, 64
    canvas = torch.zeros((L, K), device=DEV)
    # 200 rows of 64 super-blocks: 13 * 64 * 5120 bytes of records, beyond 4 MiB
    idx = _t(np.arange(200, dtype=np.int32))
    packed = torch.zeros(dq.packed_size(type_, N, K), dtype=torch.uint8, device=DEV)
    y = torch.full((200, N), -3.0, device=DEV)
    assert _call(dq, type_, canvas, idx, packed, N, y, None) == dq.DQ_EWORKSPACE
    torch.cuda.synchronize()
    assert torch.all(y == -3.0)
