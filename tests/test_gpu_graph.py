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


def test_graph_replays_of_the_next_rows(dq):
    """The fused producers, the sampler statistics, canvas attention and the
    embedding rows captured together; every replay equals the eager result."""
    L, K, F, V, M = 64, 512, 768, 20000, 6
    H, Hkv, D = 4, 2, 128
    rng = np.random.default_rng(31)
    x = _t(synth.activations(rng, L, K))
    gamma = _t((1.0 + 0.1 * rng.standard_normal(K)).astype(np.float32))
    gu = _t(synth.activations(rng, L, 2 * F))
    idx = _t(np.array([3, 60, 3, 17, 0, 41], np.int32))
    Wv = synth.q6k_weights(np.random.default_rng(32), V, K)
    pv = dq.repack_weights(dq.Q6_K, V, K, _t(Wv.reshape(-1)))
    qkv = _t(synth.qkv_rows(rng, L, H, Hkv, D))
    tab = _t(synth.rope_table(L, D, 10000.0))
    table = _t(synth.q5k_weights(np.random.default_rng(33), 50, K).reshape(-1))
    ids = _t(np.array([7, 0, 49, 7], np.int32))

    a1 = torch.empty(dq.act_size(L, K), dtype=torch.uint8, device=DEV)
    a2 = torch.empty(dq.act_size(L, F), dtype=torch.uint8, device=DEV)
    tok = torch.empty(M, dtype=torch.int32, device=DEV)
    st = torch.empty((M, 4), device=DEV)
    wss = torch.empty(dq.qgemm_rows_sample_workspace(M, V, K), dtype=torch.uint8, device=DEV)
    att = torch.empty((L, H * D), device=DEV)
    wsa = torch.empty(dq.attention_workspace(L, H, Hkv, D), dtype=torch.uint8, device=DEV)
    emb = torch.empty((ids.numel(), K), device=DEV)
    fl = torch.empty(ids.numel(), dtype=torch.int32, device=DEV)

    def step():
        dq.rmsnorm_quantize_act(x, gamma, 1e-5, out=a1)
        dq.swiglu_quantize_act(gu, F, out=a2)
        dq.qgemm_rows_sample(dq.Q6_K, x, idx, pv, V, 0.25, token=tok, stats=st, ws=wss)
        dq.attention(qkv, H, Hkv, D, tab, dq.ROPE_NEOX, out=att, ws=wsa)
        dq.embed_rows(dq.Q5_K, table, K, ids, out=emb, flags=fl)

    outs = (a1, a2, tok, st, att, emb, fl)
    step()
    torch.cuda.synchronize()
    eager = [t.clone() for t in outs]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for i in range(3):
        for t in outs:
            t.zero_() if t.dtype in (torch.uint8, torch.int32) else t.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for got, want in zip(outs, eager):
            assert torch.equal(got, want), f"replay {i} differs from the eager result"
        dq.attention(qkv, H, Hkv, D, tab, dq.ROPE_NORM)  # the program's own eager work
        torch.cuda.synchronize()


def test_graph_replays_of_the_step_at_llada_shapes(dq):
    """The benchmark's layer at L = 160 (the shared-record kernel plain and with
    the SwiGLU epilogue, the canvas kernel for down, both producers) captured
    once; every replay equals the eager result bit for bit."""
    print("graph replay of one LLaDA-8B layer at L = 160", flush=True)
    L, K, F = 160, 4096, 12288
    rng = np.random.default_rng(31)
    x = _t(synth.activations(rng, L, K))
    gamma = _t((1.0 + 0.1 * rng.standard_normal(K)).astype(np.float32))
    Wqkv = synth.q4k_weights(np.random.default_rng(32), 3 * K, K)
    gate = synth.q4k_weights(np.random.default_rng(33), F, K)
    up = synth.q4k_weights(np.random.default_rng(34), F, K)
    Wd = synth.q6k_weights(np.random.default_rng(35), K, F)
    pqkv = dq.repack_weights(dq.Q4_K, 3 * K, K, _t(Wqkv.reshape(-1)))
    pgu = dq.repack_weights(dq.Q4_K, 2 * F, K, _t(dq.interleave_gate_up(gate, up).reshape(-1)))
    pd = dq.repack_weights(dq.Q6_K, K, F, _t(Wd.reshape(-1)))
    a1 = torch.empty(dq.act_size(L, K), dtype=torch.uint8, device=DEV)
    a2 = torch.empty(dq.act_size(L, F), dtype=torch.uint8, device=DEV)
    yqkv = torch.empty((L, 3 * K), device=DEV)
    h = torch.empty((L, F), device=DEV)
    yd = torch.empty((L, K), device=DEV)

    def step():
        act = dq.rmsnorm_quantize_act(x, gamma, 1e-5, out=a1)
        dq.qgemm(dq.Q4_K, act, pqkv, 3 * K, y=yqkv)
        dq.qgemm_swiglu(dq.Q4_K, act, pgu, F, h=h)
        dq.qgemm(dq.Q6_K, dq.quantize_act(h, out=a2), pd, K, y=yd)

    outs = (yqkv, h, yd)
    step()
    torch.cuda.synchronize()
    eager = [t.clone() for t in outs]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for i in range(3):
        for t in outs:
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for got, want in zip(outs, eager):
            assert torch.equal(got, want), f"replay {i} differs from the eager result"
        dq.qgemm(dq.Q4_K, dq.quantize_act(x), pqkv, 3 * K)  # the program's own eager work
        torch.cuda.synchronize()
