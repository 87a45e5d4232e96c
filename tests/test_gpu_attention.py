"""Canvas attention on the GPU (dq_attention through the C ABI) against the oracle.

The oracle (oracle.attention) rotates Q and K with the same binary32 operation
sequence and rounds Q, K and V to binary16 exactly as the kernel does, so both
sides contract the same binary16 operands; it then works in binary64.  The
kernel accumulates in binary32 and feeds the probabilities to the second
product as binary16, so every output must lie within ATT_TOL * tol of the
oracle's, where tol[l, d] = sum_j p_j |v_j[d]| / sum_j p_j: the probabilities'
binary16 rounding (relative 2^-11 each) moves the output by at most
2^-11 * tol, the binary32 sums over at most 512 keys by about 3e-5 * tol, and
ATT_TOL = 1e-3 leaves a factor 2 over their sum.

Shapes: LLaDA-8B (L = 160, 32 heads, NORM RoPE, theta 5e5) and Dream-7B
(L = 512, 28 query heads over 4 kv heads, NEOX RoPE, theta 1e6) canvases; a
single position; a block and one key; ragged L with strided input and output
rows, no RoPE; an unaligned output (element stores); peaked scores (where a
binary16 rounding difference in a rotated element shows); every workgroup
numbering (groups of 1, 3, 4, 8, 16 and 32 query heads per kv head, and 1, 2,
3, 4, 8, 32, 64 kv heads).
"""
import numpy as np
import pytest

import oracle
import synth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

DEV = "cuda:0"
ATT_TOL = 1e-3


@pytest.fixture(scope="module")
def dq():
    import quantized_gemm_diffusion_amd as m
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    m.load_library()
    return m


def _t(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def _run(dq, L, H, Hkv, mode, theta=10000.0, scale=1.0, seed=0, pad_in=0, pad_out=0,
         out_offset=0):
    D = 128
    rng = np.random.default_rng(seed)
    width = (H + 2 * Hkv) * D
    buf = np.zeros((L, width + pad_in), np.float32)
    buf[:, :width] = synth.qkv_rows(rng, L, H, Hkv, D, scale)
    tab = synth.rope_table(L, D, theta) if mode else None
    qkv = _t(buf)
    ldo = H * D + pad_out
    out_buf = torch.full((L * ldo + out_offset + 4,), float("nan"), dtype=torch.float32,
                         device=DEV)
    out = out_buf[out_offset:out_offset + L * ldo].view(L, ldo)
    dq.attention(qkv, H, Hkv, D, _t(tab) if mode else None, mode, out=out)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    ref, tol = oracle.attention(buf[:, :width], H, Hkv, D, tab, mode)
    err = np.abs(got[:, :H * D].astype(np.float64) - ref)
    bad = err > ATT_TOL * tol
    assert not bad.any(), f"{bad.sum()} outputs out of tolerance, worst err/tol " \
                          f"{np.max(err / np.maximum(tol, 1e-300)):.3g}"
    if pad_out:
        assert np.isnan(got[:, H * D:]).all(), "padding columns written"
    tail = out_buf[out_offset + L * ldo:].cpu().numpy()
    assert np.isnan(tail).all(), "wrote past the output"
    worst = np.max(err / np.maximum(tol, 1e-300))
    print(f"attention L={L} H={H} Hkv={Hkv} mode={mode}: worst err/tol {worst:.3g}")
    return worst


def test_attention_llada_canvas(dq):
    _run(dq, 160, 32, 32, oracle.ROPE_NORM, theta=500000.0, seed=1)


def test_attention_dream_canvas(dq):
    _run(dq, 512, 28, 4, oracle.ROPE_NEOX, theta=1000000.0, seed=2)


@pytest.mark.parametrize("L", [1, 2, 33])
def test_attention_short_canvases(dq, L):
    _run(dq, L, 4, 2, oracle.ROPE_NORM, seed=10 + L)


def test_attention_ragged_strided_no_rope(dq):
    _run(dq, 77, 6, 3, oracle.ROPE_NONE, seed=3, pad_in=12, pad_out=8)


def test_attention_unaligned_output(dq):
    _run(dq, 50, 4, 4, oracle.ROPE_NEOX, seed=4, out_offset=1)


def test_attention_peaked_scores(dq):
    _run(dq, 96, 8, 2, oracle.ROPE_NORM, scale=4.0, seed=5)


@pytest.mark.parametrize("L,H,Hkv", [
    (300, 64, 8),    # groups of 8 heads: 8 heads x 2 query tiles per workgroup
    (70, 6, 2),      # groups of 3: the 4-head shape with one idle head
    (40, 32, 2),     # groups of 16: 16 heads x 1 query tile
    (45, 64, 2),     # groups of 32: two workgroups per group
    (60, 8, 8),      # no sharing, 4 query tiles: the 4-tile shape
    (200, 8, 4),     # groups of 2 over a longer canvas
    (256, 4, 1),     # 8 whole key blocks, one kv head for all
    (257, 4, 4),     # one key into a ninth block
])
def test_attention_workgroup_shapes(dq, L, H, Hkv):
    _run(dq, L, H, Hkv, oracle.ROPE_NEOX, seed=6 + H)


def test_attention_deterministic(dq):
    rng = np.random.default_rng(7)
    L, H, Hkv, D = 160, 32, 32, 128
    qkv = _t(synth.qkv_rows(rng, L, H, Hkv, D))
    tab = _t(synth.rope_table(L, D, 500000.0))
    a = dq.attention(qkv, H, Hkv, D, tab, oracle.ROPE_NORM)
    b = dq.attention(qkv, H, Hkv, D, tab, oracle.ROPE_NORM)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
