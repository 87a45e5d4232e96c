"""The hot path captured in a HIP graph (as the benchmark runs it): every
replay, with the program's own eager work and synchronizations between
replays, must equal the eager result bit for bit."""
import numpy as np
import pytest

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


def test_graph_replays_match_eager(dq):
    M, K, N, L = 40, 1024, 300, 48
    rng = np.random.default_rng(21)
    x = _t(synth.activations(rng, M, K))
    canvas = _t(synth.activations(rng, L, K))
    idx = _t(np.array([5, 47, 0, 5, 20], np.int32))
    W4 = synth.q4k_weights(np.random.default_rng(22), N, K)
    W6 = synth.q6k_weights(np.random.default_rng(23), N, K)
    p4 = dq.repack_weights(dq.Q4_K, N, K, _t(W4.reshape(-1)))
    p6 = dq.repack_weights(dq.Q6_K, N, K, _t(W6.reshape(-1)))
    abuf = torch.empty(dq.act_size(M, K), dtype=torch.uint8, device=DEV)
    y4 = torch.empty((M, N), device=DEV)
    y6 = torch.empty((M, N), device=DEV)
    yr = torch.empty((idx.numel(), N), device=DEV)
    ws = torch.empty(dq.qgemm_rows_workspace(idx.numel(), K), dtype=torch.uint8, device=DEV)

    def step():
        act = dq.quantize_act(x, out=abuf)
        dq.qgemm(dq.Q4_K, act, p4, N, y=y4)
        dq.qgemm(dq.Q6_K, act, p6, N, y=y6)
        dq.qgemm_rows(dq.Q6_K, canvas, idx, p6, N, y=yr, ws=ws)

    step()
    torch.cuda.synchronize()
    eager = [t.clone() for t in (y4, y6, yr)]

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for i in range(3):
        for t in (y4, y6, yr):
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for got, want in zip((y4, y6, yr), eager):
            assert torch.equal(got, want), f"replay {i} differs from the eager result"
        # eager work of the program's own between replays
        dq.qgemm(dq.Q4_K, dq.quantize_act(canvas), p4, N)
        torch.cuda.synchronize()
