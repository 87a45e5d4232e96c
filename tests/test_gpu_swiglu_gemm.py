"""Parity of dq_qgemm_swiglu: the stacked gate/up GEMM over tile-interleaved
weights with silu(gate) * up formed in its epilogue.

The epilogue's values are defined as the binary32 SwiGLU steps applied to the
f32 values dq_qgemm computes on the same interleaved matrix.  Checks:
  * every element of h against oracle.silu_mul of the library's own GEMM
    output, bit for bit, where the oracle's per-element loop finishes in
    seconds, else a seeded sample of 4,096;
  * dq_quantize_act(h) against oracle.swiglu_quantize_act of the GEMM output
    rearranged to [gate | up], codes, scales and sums byte for byte (the
    codes the down projection reads, as dq_swiglu_quantize_act would make
    them);
  * h against silu(g) * u of the oracle's own f64 gate and up outputs, within
    the bound that the GEMM's tolerance implies (independent of the library's
    GEMM output).
Shapes: LLaDA-8B's 160 x 12288 x 4096 and the three shared-record shapes
(on a 256-CU device; one with a last workgroup of a single tile pair), Dream-7B's
512 x 18944 x 3584 (the canvas kernel), few rows (no narrow kernel for this
call), ragged M, an odd number of tile pairs, both block types, strided h.
"""
import numpy as np
import pytest

import oracle
import synth
import act_layout

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu
DEV = "cuda:0"
TOL = 1e-4  # the GEMM's bound: |y - y_ref| <= TOL * T


@pytest.fixture(scope="module")
def dq():
    import quantized_gemm_diffusion_amd as m
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    m.load_library()
    return m


def _t(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def _deinterleave(y, F):
    """[M, 2F] output of the interleaved matrix -> [M, 2F] as [gate | up]."""
    M = y.shape[0]
    t = y.reshape(M, F // 16, 2, 16)
    return np.concatenate([t[:, :, 0, :].reshape(M, F), t[:, :, 1, :].reshape(M, F)], axis=1)


# (type, M, F, K, h row padding)
CASES = [
    (oracle.Q4_K, 160, 12288, 4096, 0),
    (oracle.Q4_K, 512, 18944, 3584, 0),
    (oracle.Q6_K, 200, 1024, 768, 0),
    (oracle.Q4_K, 20, 512, 512, 0),
    (oracle.Q4_K, 37, 592, 1280, 5),
    (oracle.Q6_K, 150, 9616, 1024, 0),
    (oracle.Q4_K, 75, 9728, 1024, 3),
    (oracle.Q6_K, 250, 5632, 1280, 0),
]


@pytest.mark.parametrize("type_,M,F,K,pad", CASES)
def test_swiglu_epilogue_bit_exact(dq, type_, M, F, K, pad):
    print(f"gate/up SwiGLU GEMM type {type_} M {M} F {F} K {K} pad {pad}", flush=True)
    rng = np.random.default_rng(M + F + K)
    gate = synth.weights(rng, type_, F, K)
    up = synth.weights(rng, type_, F, K)
    W = dq.interleave_gate_up(gate, up)
    x = synth.activations(np.random.default_rng(7 * M + K), M, K)
    act = dq.quantize_act(_t(x))
    packed = dq.repack_weights(type_, 2 * F, K, _t(W.reshape(-1)))
    hbig = torch.full((M, F + pad), -7.0, device=DEV)
    dq.qgemm_swiglu(type_, act, packed, F, h=hbig)
    y = dq.qgemm(type_, act, packed, 2 * F)
    torch.cuda.synchronize()
    hb = hbig.cpu().numpy()
    if pad:
        assert np.all(hb[:, F:] == -7.0), "stores past column F"
    h = np.ascontiguousarray(hb[:, :F])
    gu = _deinterleave(y.cpu().numpy(), F)
    g, u = gu[:, :F], gu[:, F:]
    if M * F <= 60000:
        ref = oracle.silu_mul(g, u).reshape(M, F)
        assert np.array_equal(h.view(np.uint32), ref.astype(np.float32).view(np.uint32))
    else:
        r2 = np.random.default_rng(11)
        mi, fi = r2.integers(0, M, 4096), r2.integers(0, F, 4096)
        ref = oracle.silu_mul(g[mi, fi], u[mi, fi]).astype(np.float32)
        assert np.array_equal(h[mi, fi].view(np.uint32), ref.view(np.uint32))
    if F % 256 == 0:
        q, d, b = oracle.swiglu_quantize_act(gu, F)
        ah = dq.quantize_act(_t(h))
        gq, gd, gb, padding_ok = act_layout.unpack(ah.buf.cpu().numpy(), M, F)
        assert padding_ok
        assert np.array_equal(gq, q) and np.array_equal(gb, b)
        assert np.array_equal(gd.view(np.uint32), d.view(np.uint32))


def _silu64(g):
    return g / (1.0 + np.exp(-g))


@pytest.mark.parametrize("type_,M,F,K", [(oracle.Q4_K, 160, 12288, 4096),
                                         (oracle.Q4_K, 512, 18944, 3584),
                                         (oracle.Q6_K, 200, 1024, 768)])
def test_swiglu_epilogue_against_oracle_gemm(dq, type_, M, F, K):
    """h against silu(g) * u of the oracle's f64 gate and up outputs, at 4,096
    seeded points and the corners.  With |g' - g| <= 1e-4 Tg and |u' - u| <=
    1e-4 Tu (the GEMM bound) and |silu'| <= 1.1 everywhere:
      |h' - h| <= 1.1 (|u| + du) dg + |silu(g)| du,
    plus the binary32 rounding of the epilogue's steps (1e-6 |h|)."""
    print(f"gate/up SwiGLU GEMM against the oracle: type {type_} M {M} F {F} K {K}", flush=True)
    rng = np.random.default_rng(3 * M + F)
    gate = synth.weights(rng, type_, F, K)
    up = synth.weights(rng, type_, F, K)
    W = dq.interleave_gate_up(gate, up)
    x = synth.activations(np.random.default_rng(5 * M + K), M, K)
    xq, xd, xb = oracle.quantize_act(x)
    act = dq.Act(_t(act_layout.pack(xq, xd, xb)), M, K)
    packed = dq.repack_weights(type_, 2 * F, K, _t(W.reshape(-1)))
    h = dq.qgemm_swiglu(type_, act, packed, F)
    torch.cuda.synchronize()
    h = h.cpu().numpy()
    r2 = np.random.default_rng(17)
    mi = np.concatenate([r2.integers(0, M, 4096), [0, 0, M - 1, M - 1]])
    fi = np.concatenate([r2.integers(0, F, 4096), [0, F - 1, 0, F - 1]])
    # rows of the interleaved matrix: tile i of gate at 32i .. 32i+15, of up at 32i+16 ..
    g_row = 32 * (fi // 16) + fi % 16
    g, Tg = oracle.qgemm_ref_points(type_, xq, xd, W, mi, g_row)
    u, Tu = oracle.qgemm_ref_points(type_, xq, xd, W, mi, g_row + 16)
    ref = _silu64(g) * u
    dg, du = TOL * Tg, TOL * Tu
    bound = 1.1 * (np.abs(u) + du) * dg + np.abs(_silu64(g)) * du + 1e-6 * np.abs(ref) + 1e-30
    err = np.abs(h[mi, fi].astype(np.float64) - ref)
    assert np.all(np.isfinite(h[mi, fi]))
    assert np.all(err <= bound), f"{(err > bound).sum()} points out of bound, " \
                                 f"worst err/bound {np.max(err / bound):.3g}"
