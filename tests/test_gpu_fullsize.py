"""Parity at the workloads' full sizes: every output.

Every GEMM of the LLaDA-8B (L = 160) and Dream-7B (L = 512) projection sets
in the form the benchmark runs them (Q/K/V stacked into one matrix, gate and
up stacked into one matrix, O, down), and the gathered-row output projections
(LLaDA vocab 126,464 at M = 1, 8, 32 of 160 rows; Dream vocab 152,064 at
M = 64 of 512 rows), run through the C ABI in the launch configuration the
benchmark uses.  The quantizer (or the fused RMSNorm producer) is compared bit
for bit on the whole activation, and every output of every GEMM against the
oracle's f64 plain definition (|err| <= 1e-4 * T), the oracle threaded over
the host's cores.  Seeded random shapes over the launcher's regimes are
checked on 4,096 random outputs plus one output in every (16-row block,
16-column tile) pair, or in full where the oracle finishes in seconds.
"""
import numpy as np
import pytest

import act_layout
import oracle
import synth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu
DEV = "cuda:0"
TOL = 1e-4
SAMPLES = 4096
NAMES = ["q", "k", "v", "o", "gate", "up", "down"]


@pytest.fixture(scope="module")
def dq():
    import quantized_gemm_diffusion_amd as m
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    m.load_library()
    return m


def _t(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def _full_check(type_, xq, xd, W, y, what):
    N = y.shape[1]
    assert np.all(np.isfinite(y)), what
    yr, T = oracle.qgemm_ref(type_, xq, xd, W, N)
    err = np.abs(y.astype(np.float64) - yr)
    bad = err > TOL * T
    assert not bad.any(), f"{what}: {bad.sum()} of {bad.size} outputs out of tolerance, " \
                          f"worst err/T {np.max(err / np.maximum(T, 1e-300)):.3g}"


def _sampled_check(type_, xq, xd, W, y, seed, what):
    """4,096 random outputs, the four corners, and one output in every
    (16-row block, 16-column tile) pair."""
    M, N = y.shape
    rng = np.random.default_rng(seed)
    mb, nt = (M + 15) // 16, (N + 15) // 16
    bm, bn = np.meshgrid(np.arange(mb), np.arange(nt), indexing="ij")
    tm = np.minimum(bm.ravel() * 16 + rng.integers(0, 16, bm.size), M - 1)
    tn = np.minimum(bn.ravel() * 16 + rng.integers(0, 16, bn.size), N - 1)
    mi = np.concatenate([[0, M - 1, 0, M - 1], rng.integers(0, M, SAMPLES), tm])
    ni = np.concatenate([[0, N - 1, N - 1, 0], rng.integers(0, N, SAMPLES), tn])
    yr, T = oracle.qgemm_ref_points(type_, xq, xd, W, mi, ni)
    err = np.abs(y[mi, ni].astype(np.float64) - yr)
    assert np.all(np.isfinite(y)), what
    assert np.all(err <= TOL * T), f"{what}: worst err/T {np.max(err / T):.3g}"


def _quantized(dq, M, K, seed):
    x = synth.activations(np.random.default_rng(seed), M, K)
    xq, xd, xb = oracle.quantize_act(x)
    act = dq.quantize_act(_t(x))
    q, d, b, padding_ok = act_layout.unpack(act.buf.cpu().numpy(), M, K)
    assert padding_ok
    assert np.array_equal(q, xq) and np.array_equal(b, xb)
    assert np.array_equal(d.view(np.uint32), xd.view(np.uint32))
    return xq, xd, act


def _stacked(layer_projs, config, layer, names):
    return np.concatenate([synth.weights(np.random.default_rng(synth.seed(config, layer,
                                                                          NAMES.index(n))),
                                         layer_projs[n][1], layer_projs[n][2], layer_projs[n][3])
                           for n in names])


@pytest.mark.parametrize("which", ["qkv", "o", "down_q6k", "down_q4k"])
def test_llada_projection_full_size(dq, which):
    layer = 0 if which == "down_q4k" else 1  # layer 1: down is Q6_K
    projs = {p[0]: p for p in synth.llada_layer(layer)}
    M = synth.LLADA["L"]
    if which == "qkv":
        type_, K = oracle.Q4_K, projs["q"][3]
        W = _stacked(projs, 1, layer, ["q", "k", "v"])
    else:
        name = "o" if which == "o" else "down"
        _, type_, N, K = projs[name]
        W = synth.weights(np.random.default_rng(synth.seed(1, layer, NAMES.index(name))),
                          type_, N, K)
    N = W.shape[0]
    xq, xd, act = _quantized(dq, M, K, 1000 + K + layer)
    packed = dq.repack_weights(type_, N, K, _t(W.reshape(-1)))
    y = dq.qgemm(type_, act, packed, N).cpu().numpy()
    _full_check(type_, xq, xd, W, y, f"LLaDA {which} {M}x{N}x{K}")


def test_llada_stacked_gate_up_full_size(dq):
    # the benchmark's dominant GEMM: gate and up of a layer stacked into one 24576 x 4096 Q4_K
    # matrix, its input made by the RMSNorm producer
    projs = {p[0]: p for p in synth.llada_layer(0)}
    W = _stacked(projs, 1, 0, ["gate", "up"])
    N, K = W.shape[0], projs["gate"][3]
    M = synth.LLADA["L"]
    x = synth.activations(np.random.default_rng(1100), M, K)
    gamma = (1.0 + 0.1 * np.random.default_rng(1101).standard_normal(K)).astype(np.float32)
    xq, xd, xb = oracle.rmsnorm_quantize_act(x, gamma, 1e-5)
    act = dq.rmsnorm_quantize_act(_t(x), _t(gamma), 1e-5)
    q, d, b, padding_ok = act_layout.unpack(act.buf.cpu().numpy(), M, K)
    assert padding_ok and np.array_equal(q, xq) and np.array_equal(b, xb)
    assert np.array_equal(d.view(np.uint32), xd.view(np.uint32))
    packed = dq.repack_weights(oracle.Q4_K, N, K, _t(W.reshape(-1)))
    y = dq.qgemm(oracle.Q4_K, act, packed, N).cpu().numpy()
    _full_check(oracle.Q4_K, xq, xd, W, y, "LLaDA stacked gate/up")


@pytest.mark.parametrize("which", ["qkv", "o", "gate_up", "down"])
def test_dream_projection_full_size(dq, which):
    projs = {p[0]: p for p in synth.dream_layer()}
    M = synth.DREAM["L"]
    if which in ("qkv", "gate_up"):
        names = ["q", "k", "v"] if which == "qkv" else ["gate", "up"]
        type_, K = oracle.Q4_K, projs[names[0]][3]
        W = _stacked(projs, 4, 0, names)
    else:
        _, type_, N, K = projs[which]
        W = synth.weights(np.random.default_rng(synth.seed(4, 0, NAMES.index(which))),
                          type_, N, K)
    N = W.shape[0]
    xq, xd, act = _quantized(dq, M, K, 4000 + K)
    packed = dq.repack_weights(type_, N, K, _t(W.reshape(-1)))
    y = dq.qgemm(type_, act, packed, N).cpu().numpy()
    _full_check(type_, xq, xd, W, y, f"Dream {which} {M}x{N}x{K}")


@pytest.mark.parametrize("model,Ms", [("llada", (1, 8, 32)), ("dream", (64,))])
def test_logits_rows_full_size(dq, model, Ms):
    cfg = synth.LLADA if model == "llada" else synth.DREAM
    L, K, V = cfg["L"], cfg["K"], cfg["vocab"]
    rng = np.random.default_rng(3 if model == "llada" else 5)
    canvas = synth.activations(rng, L, K)
    W = synth.q6k_weights(np.random.default_rng(synth.seed(3, 0, 7)), V, K)
    packed = dq.repack_weights(oracle.Q6_K, V, K, _t(W.reshape(-1)))
    ct = _t(canvas)
    for M in Ms:
        idx = synth.row_index(np.random.default_rng(100 + M), L, M)
        y, ws = dq.qgemm_rows(oracle.Q6_K, ct, _t(idx), packed, V)
        yn = y.cpu().numpy()
        assert not ws[: 4 * M].view(torch.int32).cpu().numpy().any()
        gq, gd, _ = oracle.qgemm_rows_inputs(canvas, idx)
        _full_check(oracle.Q6_K, gq, gd, W, yn, f"{model} logits M={M}")


def _random_shapes(count, seed):
    """Seeded shapes spread over the launcher's regimes: narrow and few-row
    kernels (M <= 32, 8 to 16 super-blocks, wide N), the canvas kernel with two
    or three n-tiles per wave and 2-, 4- or 8-wave workgroups, ragged M and N."""
    rng = np.random.default_rng(seed)
    shapes = []
    for i in range(count):
        type_ = oracle.Q4_K if rng.integers(2) == 0 else oracle.Q6_K
        if i % 3 == 0:      # narrow / single-row / few-row: M <= 32, nb even in [8, 16]
            M = int(rng.choice([1, 2, 3, 4, 7, 16, 23, 32]))
            nb = int(rng.choice([8, 10, 12, 14, 16]))
            N = int(rng.integers(16384, 40000))
        else:               # canvas kernel
            M = int(rng.integers(33, 600))
            nb = int(rng.choice([1, 2, 3, 5, 14, 16, 20, 48]))
            N = int(rng.integers(17, 30000))
        shapes.append((type_, M, N, 256 * nb))
    return shapes


@pytest.mark.parametrize("type_,M,N,K", _random_shapes(12, 2024))
def test_random_shapes(dq, type_, M, N, K):
    W = synth.weights(np.random.default_rng(M * 7 + N), type_, N, K)
    x = synth.activations(np.random.default_rng(M + N), M, K)
    xq, xd, _ = oracle.quantize_act(x)
    act = dq.quantize_act(_t(x))
    packed = dq.repack_weights(type_, N, K, _t(W.reshape(-1)))
    y = dq.qgemm(type_, act, packed, N).cpu().numpy()
    what = f"type {type_} {M}x{N}x{K}"
    if M * N * K <= 4_000_000_000:
        _full_check(type_, xq, xd, W, y, what)
    else:
        _sampled_check(type_, xq, xd, W, y, 13, what)
