"""Embedding rows on the GPU (dq_embed_rows through the C ABI) against the oracle.

Every decoded value is bit-exact: both sides form the correctly rounded
binary32 of each type's definition (the oracle in binary64, where every
product is exact, then one rounding).  Tables are seeded random bytes in each
GGUF layout (F32, F16, BF16, Q8_0, Q4_K, Q5_K, Q6_K); ids include duplicates,
any order and out-of-range values (a zero row and a flag); outputs strided
(padding untouched) and unaligned (element stores).  The LLaDA-8B token table
(126,464 x 4096 Q4_K) is decoded on the 160 rows of a canvas.
"""
import numpy as np
import pytest

import oracle
import synth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

DEV = "cuda:0"
TYPES = [synth.F32, synth.F16, synth.BF16, synth.Q8_0, synth.Q4_K, synth.Q5_K, synth.Q6_K]


@pytest.fixture(scope="module")
def dq():
    import quantized_gemm_diffusion_amd as m
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    m.load_library()
    return m


def _t(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


@pytest.mark.parametrize("type_", TYPES)
def test_embed_rows_bit_exact(dq, type_):
    rng = np.random.default_rng(100 + type_)
    N, K = 37, 768
    table = synth.table(rng, type_, N, K)
    ids = np.array([5, 0, 36, 5, 12, -1, 37, 20, 36, 1 << 30], np.int32)
    out, flags = dq.embed_rows(type_, _t(table.reshape(-1)), K, _t(ids))
    torch.cuda.synchronize()
    ref, rflag = oracle.embed_rows(type_, table, K, ids)
    got = out.cpu().numpy()
    assert np.array_equal(flags.cpu().numpy(), rflag)
    fin = np.isfinite(ref)
    assert np.array_equal(got[fin].view(np.uint32), ref[fin].view(np.uint32))
    assert np.array_equal(np.isnan(got), np.isnan(ref))


@pytest.mark.parametrize("type_", [synth.Q4_K, synth.Q6_K, synth.BF16])
def test_embed_rows_strided_and_unaligned(dq, type_):
    rng = np.random.default_rng(200 + type_)
    N, K, M = 19, 512, 7
    table = synth.table(rng, type_, N, K)
    ids = rng.integers(0, N, M).astype(np.int32)
    ref, _ = oracle.embed_rows(type_, table, K, ids)
    # strided: padding columns keep their NaN
    buf = torch.full((M, K + 12), float("nan"), dtype=torch.float32, device=DEV)
    dq.embed_rows(type_, _t(table.reshape(-1)), K, _t(ids), out=buf[:, :K])
    got = buf.cpu().numpy()
    assert np.array_equal(got[:, :K].view(np.uint32), ref.view(np.uint32))
    assert np.isnan(got[:, K:]).all()
    # unaligned rows (4-byte offset): element stores
    flat = torch.full((M * K + 8,), float("nan"), dtype=torch.float32, device=DEV)
    view = flat[1:1 + M * K].view(M, K)
    dq.embed_rows(type_, _t(table.reshape(-1)), K, _t(ids), out=view)
    got = flat.cpu().numpy()
    assert np.array_equal(got[1:1 + M * K].reshape(M, K).view(np.uint32), ref.view(np.uint32))
    assert np.isnan(got[0]) and np.isnan(got[1 + M * K:]).all()


def test_embed_rows_llada_token_table(dq):
    cfg = synth.LLADA
    N, K, L = cfg["vocab"], cfg["K"], cfg["L"]
    rng = np.random.default_rng(synth.seed(5, 0, 0))
    table = synth.q4k_weights(rng, N, K).reshape(N, -1)
    ids = rng.integers(0, N, L).astype(np.int32)
    out, flags = dq.embed_rows(synth.Q4_K, _t(table.reshape(-1)), K, _t(ids))
    torch.cuda.synchronize()
    ref, _ = oracle.embed_rows(synth.Q4_K, table, K, ids)
    assert not flags.cpu().numpy().any()
    assert np.array_equal(out.cpu().numpy().view(np.uint32), ref.view(np.uint32))
