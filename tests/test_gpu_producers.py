"""GPU parity of the fused producers (SwiGLU -> quantize, RMSNorm -> quantize)
against the oracle: codes, scales and code sums bit for bit, on ragged and
full-size shapes, contiguous and strided (unaligned) rows, and inputs at the
edges of the defined exponential's range."""
import numpy as np
import pytest

import act_layout
import oracle

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


def _same(act, ref, M, K):
    q, d, b, padding_ok = act_layout.unpack(act.buf.cpu().numpy(), M, K)
    rq, rd, rb = ref
    assert padding_ok
    assert np.array_equal(q, rq), f"codes differ in {np.count_nonzero(q != rq)} places"
    assert np.array_equal(d.view(np.uint32), rd.view(np.uint32)), "scales differ"
    assert np.array_equal(b, rb), "code sums differ"


def _gu(rng, M, F, pad=0):
    gu = np.zeros((M, 2 * F + pad), np.float32)
    gu[:, :F] = rng.normal(0, 3, (M, F))
    gu[:, F:2 * F] = rng.normal(0, 1, (M, F))
    # the exponential's clamps and large/small arguments, and exact zeros
    edge = np.float32([0.0, -0.0, 87.5, -87.5, 100.0, -100.0, 88.0, -87.0, 1e-30, -1e-30])
    gu[0, :edge.size] = edge
    gu[-1, F:F + 8] = 0.0
    return gu


@pytest.mark.parametrize("M,F,pad", [(1, 256, 0), (37, 512, 0), (20, 768, 3), (160, 12288, 0)])
def test_swiglu_quantize_bit_exact(dq, M, F, pad):
    rng = np.random.default_rng(100 + M + pad)
    gu = _gu(rng, M, F, pad)
    ref = oracle.swiglu_quantize_act(gu, F)
    act = dq.swiglu_quantize_act(_t(gu), F)
    torch.cuda.synchronize()
    _same(act, ref, M, F)


@pytest.mark.parametrize("M,K,pad,eps", [(1, 256, 0, 1e-5), (37, 512, 0, 0.0), (20, 768, 3, 1e-6),
                                         (160, 4096, 0, 1e-5), (17, 12288, 0, 1e-5),
                                         (5, 3584, 0, 1e-5),   # fewer blocks than waves
                                         (512, 3584, 0, 1e-5),  # Dream-7B's canvas
                                         (2, 262144, 0, 1e-5)])  # the largest K: 64 blocks a wave
def test_rmsnorm_quantize_bit_exact(dq, M, K, pad, eps):
    rng = np.random.default_rng(200 + M + pad)
    x = np.zeros((M, K + pad), np.float32)
    x[:, :K] = rng.normal(0, 1, (M, K))
    x[0, :K] = 0.0                       # an all-zero row: rinv = 1/sqrt(eps) or inf * 0
    if eps == 0.0:
        x[0, 0] = 1.0                    # keep the row finite when eps = 0
    x[-1, :K:97] *= 20.0                 # outlier channels
    gamma = rng.normal(1, 0.2, K).astype(np.float32)
    ref = oracle.rmsnorm_quantize_act(x[:, :K], gamma, eps)
    xt = _t(x)[:, :K] if pad else _t(x)
    act = dq.rmsnorm_quantize_act(xt, _t(gamma), eps)
    torch.cuda.synchronize()
    _same(act, ref, M, K)


def test_swiglu_output_feeds_the_gemm(dq):
    """The stacked gate/up GEMM's output goes straight into the down projection's quantizer."""
    import synth
    M, K, F = 48, 512, 768
    rng = np.random.default_rng(300)
    W = synth.q4k_weights(rng, 2 * F, K)
    x = synth.activations(rng, M, K)
    act = dq.quantize_act(_t(x))
    packed = dq.repack_weights(oracle.Q4_K, 2 * F, K, _t(W.reshape(-1)))
    gu = dq.qgemm(oracle.Q4_K, act, packed, 2 * F)
    down_in = dq.swiglu_quantize_act(gu, F)
    torch.cuda.synchronize()
    _same(down_in, oracle.swiglu_quantize_act(gu.cpu().numpy(), F), M, F)
