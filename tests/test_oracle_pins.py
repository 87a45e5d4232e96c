"""Pins of the CPU oracle to things other than itself (CPU only).

* fp16 decode: exhaustive against numpy's float16 (an independent library).
* Q4_K / Q6_K decode: hand-built golden blocks (tests/golden), every 6-bit
  scale/min value in every slot, and a round trip against the field-level
  encoder in kq_fields.py (written per weight position, the inverse map).
* Activation quantization: closed forms (amax -> +-127, integer identity,
  half-way ties to even, the rounding-error bound, zero blocks, sign and
  power-of-two scaling symmetry, bsum as a plain integer sum).
* Sub-block dots and per-super-block sums: numpy int64 brute force straight
  from the fields; with unit scales the sums reduce to numpy.matmul.
* Reference GEMM: numpy float64 brute force from the fields; the oracle's own
  f32 output through the integer decomposition lies within 1e-6 * T.
* Fused producers: the defined exp within 2 ulp of numpy's float64 exp over
  its range (and its clamps), SiLU times up against float64, SwiGLU and
  RMSNorm closed forms (exact codes for integer inputs), exact power-of-two
  scaling invariance, and RMSNorm against the float64 formula within the
  quantizer's rounding.
* Sampler statistics of the logits: closed forms (uniform and two-level
  rows), scipy's logsumexp and entropy on random rows, the first index on
  ties, the binary32 product deciding the token, exact power-of-two
  temperature and integer shift invariance, and no overflow at large
  magnitudes.
* Attention: binary32 -> binary16 rounding against numpy's float16 at every
  rounding boundary of every exponent (and random patterns); RoPE against complex multiplication in float64 for both pairings
  (and exact special angles); attention closed forms (one position, equal
  keys, constant values, two keys), permutation equivariance, shared kv heads,
  and rotation invariance of the scores (RoPE depends on relative position).
* The decoder's other types: binary16 exhaustively against numpy; bfloat16 on
  exact constants and on every binary32 whose low half is zero; Q8_0 and Q5_K
  on hand-built blocks with closed-form values (every code, the fifth bit in
  every chunk) and on random fields through the per-weight encoder; embedding
  rows equal to the decoded rows they select, out-of-range ids flagged.
"""
import os

import numpy as np
import pytest

import oracle
from kq_fields import (dequant_q4k_fields, dequant_q6k_fields, enc_q4k, enc_q6k,
                       encode_q4k_matrix, encode_q6k_matrix, random_q4k_fields,
                       random_q6k_fields)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _read_golden(name):
    out = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            if line.startswith("#") or ":" not in line:
                continue
            k, v = line.split(":", 1)
            out[k.strip()] = v.split()
    return out


# --------------------------------------------------------------------------- #
# fp16                                                                        #
# --------------------------------------------------------------------------- #
def test_fp16_exhaustive_against_numpy():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = oracle.fp16_to_f32(bits)
    ref = bits.view(np.float16).astype(np.float32)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan].view(np.uint32), ref[~nan].view(np.uint32))


# --------------------------------------------------------------------------- #
# Q4_K                                                                        #
# --------------------------------------------------------------------------- #
def test_q4k_handbuilt_golden():
    g = _read_golden("q4k_handbuilt.txt")
    blk = np.array([int(b, 16) for b in g["bytes"]], np.uint8)
    assert blk.size == 144
    d, dmin, sc, mn, q = oracle.decode_q4k(blk)
    assert d == np.float32(g["d"][0]) and dmin == np.float32(g["dmin"][0])
    assert list(sc) == [int(v) for v in g["sc"]]
    assert list(mn) == [int(v) for v in g["mn"]]
    exp_q = np.zeros(256, np.int64)
    for c in range(4):
        for l in range(32):
            exp_q[64 * c + l] = l % 16
            exp_q[64 * c + 32 + l] = 2 * c + l // 16
    assert np.array_equal(q.astype(np.int64), exp_q)
    w = oracle.dequant(oracle.Q4_K, blk, 256)[0]
    sc_i = np.repeat(np.array(g["sc"], np.float64), 32)
    mn_i = np.repeat(np.array(g["mn"], np.float64), 32)
    assert np.array_equal(w, 1.0 * sc_i * exp_q - 0.5 * mn_i)


@pytest.mark.parametrize("slot", range(8))
def test_q4k_every_scale_and_min_value_in_every_slot(slot):
    rng = np.random.default_rng(100 + slot)
    for v in range(64):
        sc = rng.integers(0, 64, 8)
        mn = rng.integers(0, 64, 8)
        sc[slot] = v
        mn[slot] = 63 - v
        blk = enc_q4k(1.0, 1.0, sc, mn, np.zeros(256, np.int64))
        _, _, dsc, dmn, _ = oracle.decode_q4k(blk)
        assert list(dsc) == list(sc) and list(dmn) == list(mn), (slot, v)


def test_q4k_random_round_trip():
    rng = np.random.default_rng(7)
    f = random_q4k_fields(rng, 6, 3)
    W = encode_q4k_matrix(f)
    for n in range(6):
        for b in range(3):
            d, dmin, sc, mn, q = oracle.decode_q4k(W[n, b])
            assert d == np.float32(f["d"][n, b]) and dmin == np.float32(f["dmin"][n, b])
            assert np.array_equal(sc, f["sc"][n, b]) and np.array_equal(mn, f["mn"][n, b])
            assert np.array_equal(q, f["q"][n, b])
    assert np.array_equal(oracle.dequant(oracle.Q4_K, W, 768), dequant_q4k_fields(f))


def test_q4k_negative_and_subnormal_superblock_scales():
    q = np.arange(256) % 16
    sc = np.arange(8) + 1
    mn = np.arange(8) * 3
    sub = np.float16(2.0 ** -20)  # fp16 subnormal
    blk = enc_q4k(-2.0, sub, sc, mn, q)
    d, dmin, *_ = oracle.decode_q4k(blk)
    assert d == -2.0 and dmin == np.float32(2.0 ** -20)
    w = oracle.dequant(oracle.Q4_K, blk, 256)[0]
    exp = -2.0 * np.repeat(sc, 32) * q - 2.0 ** -20 * np.repeat(mn, 32)
    assert np.array_equal(w, exp)


# --------------------------------------------------------------------------- #
# Q6_K                                                                        #
# --------------------------------------------------------------------------- #
def test_q6k_handbuilt_golden():
    g = _read_golden("q6k_handbuilt.txt")
    blk = np.zeros(210, np.uint8)
    for item in g["set"]:
        pos, val = item.split("=")
        blk[int(pos)] = int(val, 16)
    d, sc, q = oracle.decode_q6k(blk)
    assert d == np.float32(g["d"][0])
    assert list(sc) == [int(v) for v in g["sc"]]
    exp_q = np.zeros(256, np.int64)
    for item in g["q"]:
        i, v = item.split("=")
        exp_q[int(i)] = int(v)
    assert np.array_equal(q.astype(np.int64), exp_q)
    w = oracle.dequant(oracle.Q6_K, blk, 256)[0]
    sc_i = np.repeat(np.array(g["sc"], np.float64), 16)
    assert np.array_equal(w, 0.25 * sc_i * (exp_q - 32))


def test_q6k_random_round_trip_full_scale_range():
    rng = np.random.default_rng(8)
    f = random_q6k_fields(rng, 6, 3)  # scales over the whole int8 range
    W = encode_q6k_matrix(f)
    for n in range(6):
        for b in range(3):
            d, sc, q = oracle.decode_q6k(W[n, b])
            assert d == np.float32(f["d"][n, b])
            assert np.array_equal(sc, f["sc"][n, b]) and np.array_equal(q, f["q"][n, b])
    assert np.array_equal(oracle.dequant(oracle.Q6_K, W, 768), dequant_q6k_fields(f))


def test_q6k_every_code_at_every_quarter():
    # each 6-bit code value at each of the 8 (half, quarter) positions
    for h in range(2):
        for quarter in range(4):
            for l in (0, 17, 31):
                for v in range(64):
                    q = np.zeros(256, np.int64)
                    q[128 * h + 32 * quarter + l] = v
                    _, _, dq = oracle.decode_q6k(enc_q6k(1.0, np.ones(16, np.int64), q))
                    assert np.array_equal(dq, q), (h, quarter, l, v)


# --------------------------------------------------------------------------- #
# Activation quantization                                                     #
# --------------------------------------------------------------------------- #
def test_quant_amax_maps_to_127_and_scale():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((5, 512)).astype(np.float32)
    q, d, bs = oracle.quantize_act(x)
    for m in range(5):
        for b in range(2):
            blk = x[m, 256 * b:256 * (b + 1)]
            i = np.argmax(np.abs(blk))
            assert q[m, 256 * b + i] == (127 if blk[i] > 0 else -127)
            assert d[m, b] == np.float32(np.abs(blk[i])) / np.float32(127)


def test_quant_integer_identity():
    rng = np.random.default_rng(2)
    x = rng.integers(-127, 128, (3, 768)).astype(np.float32)
    x[:, ::256] = 127.0  # amax = 127 in every block
    q, d, bs = oracle.quantize_act(x)
    assert np.array_equal(q.astype(np.float32), x)
    assert np.all(d == 1.0)


def test_quant_ties_to_even():
    # amax = 254 -> inv = 0.5 exactly; x = 2k+1 lands on k + 0.5
    x = np.zeros((1, 256), np.float32)
    x[0, 0] = 254.0
    odd = np.arange(1, 254, 2, dtype=np.float32)[:120]
    x[0, 1:121] = odd
    x[0, 121:241] = -odd
    q, d, _ = oracle.quantize_act(x)
    half = odd / 2.0  # k + 0.5
    exp = np.where(np.floor(half) % 2 == 0, np.floor(half), np.ceil(half))
    assert np.array_equal(q[0, 1:121], exp.astype(np.int8))
    assert np.array_equal(q[0, 121:241], (-exp).astype(np.int8))
    assert d[0, 0] == np.float32(2.0)


def test_quant_error_bound_sign_and_scaling():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((4, 1024)).astype(np.float32) * 3
    q, d, bs = oracle.quantize_act(x)
    xhat = q.astype(np.float64) * np.repeat(d, 256, axis=1)
    bound = np.repeat(d, 256, axis=1) * 0.5 * (1 + 2.0 ** -21)
    assert np.all(np.abs(x - xhat) <= bound)
    qn, dn, bn = oracle.quantize_act(-x)
    assert np.array_equal(qn, -q) and np.array_equal(dn, d) and np.array_equal(bn, -bs)
    for k in (-7, 5):
        qs, ds, _ = oracle.quantize_act(x * np.float32(2.0 ** k))
        assert np.array_equal(qs, q) and np.array_equal(ds, d * np.float32(2.0 ** k))


def test_quant_zero_block_and_bsum():
    rng = np.random.default_rng(4)
    x = rng.standard_normal((3, 768)).astype(np.float32)
    x[1, 256:512] = 0.0
    q, d, bs = oracle.quantize_act(x)
    assert np.all(q[1, 256:512] == 0) and d[1, 1] == 0.0 and np.all(bs[1, 8:16] == 0)
    assert np.array_equal(bs, q.astype(np.int64).reshape(3, 24, 32).sum(-1))


# --------------------------------------------------------------------------- #
# Sub-block dots, per-super-block sums, GEMM                                  #
# --------------------------------------------------------------------------- #
def _q4k_case(seed, M, N, nb):
    rng = np.random.default_rng(seed)
    f = random_q4k_fields(rng, N, nb)
    W = encode_q4k_matrix(f)
    x = rng.standard_normal((M, nb * 256)).astype(np.float32)
    return f, W, x


def _q6k_case(seed, M, N, nb, sc_lo=-128, sc_hi=127):
    rng = np.random.default_rng(seed)
    f = random_q6k_fields(rng, N, nb, sc_lo, sc_hi)
    W = encode_q6k_matrix(f)
    x = rng.standard_normal((M, nb * 256)).astype(np.float32)
    return f, W, x


def test_q4k_subdots_and_sums_brute_force():
    M, N, nb = 3, 5, 2
    f, W, x = _q4k_case(11, M, N, nb)
    q, d, bs = oracle.quantize_act(x)
    dots = oracle.subdots(oracle.Q4_K, q, W, N)
    qx = q.astype(np.int64).reshape(M, nb, 8, 32)
    qw = f["q"].astype(np.int64).reshape(N, nb, 8, 32)
    exp = np.einsum("mbjk,nbjk->mnbj", qx, qw)
    assert np.array_equal(dots, exp)
    S, Mn = oracle.superblock_sums(oracle.Q4_K, q, bs, W, N)
    assert np.array_equal(S, np.einsum("mnbj,nbj->mnb", exp, f["sc"]))
    bsx = qx.sum(-1)  # [M, nb, 8]
    assert np.array_equal(Mn, np.einsum("mbj,nbj->mnb", bsx, f["mn"]))


def test_q6k_subdots_and_sums_brute_force():
    M, N, nb = 3, 5, 2
    f, W, x = _q6k_case(12, M, N, nb)
    q, d, bs = oracle.quantize_act(x)
    dots = oracle.subdots(oracle.Q6_K, q, W, N)
    qx = q.astype(np.int64).reshape(M, nb, 16, 16)
    qw = (f["q"].astype(np.int64) - 32).reshape(N, nb, 16, 16)
    exp = np.einsum("mbjk,nbjk->mnbj", qx, qw)
    assert np.array_equal(dots, exp)
    S, Mn = oracle.superblock_sums(oracle.Q6_K, q, bs, W, N)
    assert np.array_equal(S, np.einsum("mnbj,nbj->mnb", exp, f["sc"]))
    assert np.all(Mn == 0)


def test_unit_scales_reduce_to_integer_matmul():
    # d = 1, dmin = 0, sc = 1, mn = 0: sum over the row of S is q_x . q_w
    rng = np.random.default_rng(13)
    M, N, nb = 4, 6, 3
    qw = rng.integers(0, 16, (N, nb, 256))
    W = np.stack([np.stack([enc_q4k(1.0, 0.0, np.ones(8, int), np.zeros(8, int), qw[n, b])
                            for b in range(nb)]) for n in range(N)])
    x = rng.integers(-127, 128, (M, nb * 256)).astype(np.float32)
    x[:, ::256] = 127.0
    q, d, bs = oracle.quantize_act(x)
    S, _ = oracle.superblock_sums(oracle.Q4_K, q, bs, W, N)
    ref = np.matmul(q.astype(np.int64), qw.reshape(N, -1).T)
    assert np.array_equal(S.sum(-1), ref)
    y, T = oracle.qgemm_ref(oracle.Q4_K, q, d, W, N)
    assert np.array_equal(y, ref.astype(np.float64))


@pytest.mark.parametrize("kind", ["q4k", "q6k"])
def test_gemm_reference_brute_force_and_decomposition(kind):
    M, N, nb = 5, 7, 3
    if kind == "q4k":
        f, W, x = _q4k_case(21, M, N, nb)
        t, wf = oracle.Q4_K, dequant_q4k_fields(f)
    else:
        f, W, x = _q6k_case(22, M, N, nb)
        t, wf = oracle.Q6_K, dequant_q6k_fields(f)
    q, d, bs = oracle.quantize_act(x)
    xh = q.astype(np.float64) * np.repeat(d, 256, axis=1).astype(np.float64)
    y_bf = xh @ wf.T
    T_bf = np.abs(xh) @ np.abs(wf).T
    y, T = oracle.qgemm_ref(t, q, d, W, N)
    assert np.all(np.abs(y - y_bf) <= 1e-12 * T_bf)
    assert np.allclose(T, T_bf, rtol=1e-12, atol=0)
    # the integer decomposition in f64 equals the plain definition
    S, Mn = oracle.superblock_sums(t, q, bs, W, N)
    if kind == "q4k":
        dd, dm = f["d"].astype(np.float64), f["dmin"].astype(np.float64)
    else:
        dd, dm = f["d"].astype(np.float64), np.zeros_like(f["d"], np.float64)
    y_dec = np.einsum("mb,mnb->mn", d.astype(np.float64),
                      dd[None] * S - dm[None] * Mn.astype(np.float64))
    assert np.all(np.abs(y_dec - y) <= 1e-12 * T)
    # the oracle's own binary32 output
    y32 = oracle.qgemm_f32(t, q, d, bs, W, N)
    assert np.all(np.abs(y32.astype(np.float64) - y) <= 1e-6 * T)
    # sampled points agree with the dense routine
    mi = np.array([0, 4, 2]); ni = np.array([6, 0, 3])
    yp, Tp = oracle.qgemm_ref_points(t, q, d, W, mi, ni)
    assert np.array_equal(yp, y[mi, ni]) and np.array_equal(Tp, T[mi, ni])


def test_rows_inputs_gather_then_quantize():
    rng = np.random.default_rng(31)
    canvas = rng.standard_normal((20, 512)).astype(np.float32)
    idx = np.array([7, 3, 3, 19, 0], np.int32)
    q, d, bs = oracle.qgemm_rows_inputs(canvas, idx)
    qa, da, ba = oracle.quantize_act(canvas)
    assert np.array_equal(q, qa[idx]) and np.array_equal(d, da[idx]) and np.array_equal(bs, ba[idx])


# --------------------------------------------------------------------------- #
# The fused producers of the GEMM inputs (Architecture page, "A forward pass",  #
# step 2: RMSNorm, then the Q/K/V quantization; SiLU on gate times up, then the #
# down quantization).  Pinned to numpy's float64 functions, closed forms and    #
# exact scaling identities.                                                     #
# --------------------------------------------------------------------------- #
def test_exp_within_two_ulp_of_float64_over_its_range():
    t = np.concatenate([np.linspace(-87.0, 88.0, 40001, dtype=np.float32),
                        np.float32([0.0, -0.0, 1e-8, -1e-8, 0.3465, -0.3466, 87.99, -86.99])])
    e = oracle.exp_f32(t).astype(np.float64)
    ref = np.exp(t.astype(np.float64))
    assert np.all(np.abs(e - ref) <= 2.0 * 2.0 ** -23 * ref)
    assert oracle.exp_f32([0.0])[0] == 1.0
    # clamped outside [-87, 88]
    assert oracle.exp_f32([100.0])[0] == oracle.exp_f32([88.0])[0]
    assert oracle.exp_f32([-1e30])[0] == oracle.exp_f32([-87.0])[0]


def test_silu_mul_against_float64_and_closed_forms():
    rng = np.random.default_rng(11)
    g = np.concatenate([rng.normal(0, 4, 3000), [0.0, 1.0, -1.0, 30.0, -30.0, 80.0, -80.0]])
    g = g.astype(np.float32)
    u = rng.normal(0, 2, g.size).astype(np.float32)
    got = oracle.silu_mul(g, u).astype(np.float64)
    g64, u64 = g.astype(np.float64), u.astype(np.float64)
    ref = g64 / (1.0 + np.exp(-g64)) * u64
    assert np.all(np.abs(got - ref) <= 8 * 2.0 ** -24 * np.abs(ref) + 1e-37)
    assert oracle.silu_mul([0.0], [5.0])[0] == 0.0
    # for large g, 1 + e^-g rounds to 1 and silu(g) * u is g * u exactly
    assert oracle.silu_mul([50.0], [3.0])[0] == np.float32(150.0)


def test_swiglu_quantize_closed_form():
    # gate = 50 makes silu(gate) = 50 exactly; up holds integers with |max| 127,
    # so the codes are up itself and d = 50
    rng = np.random.default_rng(12)
    F = 512
    up = rng.integers(-127, 128, (3, F)).astype(np.float32)
    up[:, 0] = 127.0
    up[:, 256] = -127.0
    gu = np.concatenate([np.full((3, F), 50.0, np.float32), up], axis=1)
    q, d, b = oracle.swiglu_quantize_act(gu, F)
    assert np.array_equal(q, up.astype(np.int8))
    assert np.all(d == 50.0)
    assert np.array_equal(b, up.reshape(3, F // 32, 32).sum(axis=2).astype(np.int32))
    # up = 0 gives all-zero codes and scales
    gu0 = np.concatenate([rng.normal(0, 1, (2, F)).astype(np.float32),
                          np.zeros((2, F), np.float32)], axis=1)
    q0, d0, b0 = oracle.swiglu_quantize_act(gu0, F)
    assert not q0.any() and not d0.any() and not b0.any()


def test_rmsnorm_quantize_closed_forms_and_scaling():
    K = 1024
    rng = np.random.default_rng(13)
    gamma = rng.integers(-127, 128, K).astype(np.float32)
    gamma[0], gamma[300], gamma[600], gamma[900] = 127.0, -127.0, 127.0, -127.0
    # all-ones rows: the sum of squares is K exactly, rinv = 1 with eps = 0, y = gamma
    q, d, b = oracle.rmsnorm_quantize_act(np.ones((2, K), np.float32), gamma, 0.0)
    assert np.array_equal(q[0], gamma.astype(np.int8)) and np.all(d == 1.0)
    # with eps = 0 every step scales exactly by powers of two: 2^k x gives the same codes
    x = rng.normal(0, 1, (4, K)).astype(np.float32)
    g2 = rng.normal(1, 0.1, K).astype(np.float32)
    q1, d1, _ = oracle.rmsnorm_quantize_act(x, g2, 0.0)
    q2, d2, _ = oracle.rmsnorm_quantize_act(x * np.float32(64.0), g2, 0.0)
    assert np.array_equal(q1, q2) and np.array_equal(d1, d2)
    # the normalized values agree with the float64 formula (the codes then follow the
    # quantizer, pinned above): compare dequantized values within the code rounding
    eps = 1e-5
    q3, d3, _ = oracle.rmsnorm_quantize_act(x, g2, eps)
    x64 = x.astype(np.float64)
    y = x64 / np.sqrt(np.mean(x64 * x64, axis=1, keepdims=True) + eps) * g2.astype(np.float64)
    deq = q3.astype(np.float64) * np.repeat(d3.astype(np.float64), 256, axis=1)
    assert np.all(np.abs(deq - y) <= np.repeat(d3.astype(np.float64), 256, axis=1) * 0.5001 + 1e-6)


# --- sampler statistics of the logits ---------------------------------------

def test_logits_stats_uniform_and_two_level_closed_forms():
    N = 1000
    tok, st = oracle.logits_stats(np.full((1, N), 2.5), 1.0)
    assert tok[0] == 0
    np.testing.assert_allclose(st[0], [2.5, 2.5 + np.log(N), np.log(N), 1.0 / N], rtol=1e-13)
    # k entries at a, N - k at b
    k, a, b = 7, 3.0, -1.0
    y = np.full(N, b)
    pos = np.random.default_rng(3).choice(N, k, replace=False)
    y[pos] = a
    tok, st = oracle.logits_stats(y[None, :], 1.0)
    zsum = k * np.exp(a) + (N - k) * np.exp(b)
    pa, pb = np.exp(a) / zsum, np.exp(b) / zsum
    assert tok[0] == pos.min()
    np.testing.assert_allclose(st[0], [a, np.log(zsum), -k * pa * np.log(pa) - (N - k) * pb * np.log(pb), pa],
                               rtol=1e-12)


def test_logits_stats_against_scipy():
    from scipy.special import logsumexp, softmax
    from scipy.stats import entropy
    rng = np.random.default_rng(11)
    for scale, beta in ((1.0, 1.0), (30.0, 0.05), (0.01, 8.0)):
        y = (rng.standard_normal((5, 4099)) * scale).astype(np.float32).astype(np.float64)
        tok, st = oracle.logits_stats(y, beta)
        z = (np.float32(beta) * y.astype(np.float32)).astype(np.float64)
        np.testing.assert_array_equal(tok, np.argmax(z, axis=1))
        np.testing.assert_array_equal(st[:, 0], z.max(axis=1))
        np.testing.assert_allclose(st[:, 1], logsumexp(z, axis=1), rtol=1e-13)
        np.testing.assert_allclose(st[:, 2], entropy(softmax(z, axis=1), axis=1), rtol=1e-10, atol=1e-13)
        np.testing.assert_allclose(st[:, 3], softmax(z, axis=1).max(axis=1), rtol=1e-12)


def test_logits_stats_token_is_first_maximum_of_the_binary32_product():
    tok, _ = oracle.logits_stats(np.array([[0.0, 5.0, 2.0, 5.0, -1.0]]), 1.0)
    assert tok[0] == 1
    # 1 + 2^-30 rounds to 1.0f: a tie in binary32, so the first index wins
    tok, st = oracle.logits_stats(np.array([[1.0, 1.0 + 2.0 ** -30]]), 1.0)
    assert tok[0] == 0 and st[0, 0] == 1.0
    # 3 * 0.1f and 3 * 0.1 differ: the binary32 product is the one reported
    _, st = oracle.logits_stats(np.array([[3.0]]), 0.1)
    assert st[0, 0] == float(np.float32(3.0) * np.float32(0.1))


def test_logits_stats_temperature_and_shift_invariance():
    rng = np.random.default_rng(5)
    y = rng.integers(-200, 200, size=(4, 777)).astype(np.float64)
    t1, s1 = oracle.logits_stats(y, 0.25)
    t2, s2 = oracle.logits_stats(0.25 * y, 1.0)
    np.testing.assert_array_equal(t1, t2)
    np.testing.assert_array_equal(s1, s2)
    t3, s3 = oracle.logits_stats(y + 1000.0, 1.0)
    t4, s4 = oracle.logits_stats(y, 1.0)
    np.testing.assert_array_equal(t3, t4)
    np.testing.assert_allclose(s3[:, :2] - 1000.0, s4[:, :2], rtol=0, atol=1e-9)
    np.testing.assert_allclose(s3[:, 2:], s4[:, 2:], rtol=1e-9, atol=1e-15)


def test_logits_stats_large_magnitudes_do_not_overflow():
    tok, st = oracle.logits_stats(np.array([[1e4, 0.0, -1e4, 9990.0]]), 1.0)
    assert tok[0] == 0
    assert np.all(np.isfinite(st))
    np.testing.assert_allclose(st[0, 1], 1e4 + np.log1p(np.exp(-10.0)), rtol=1e-14)
    p = 1.0 / (1.0 + np.exp(-10.0))
    np.testing.assert_allclose(st[0, 2], -p * np.log(p) - (1 - p) * np.log(1 - p), rtol=1e-9)
    np.testing.assert_allclose(st[0, 3], p, rtol=1e-11)  # exp of a difference of ~1e4-sized values


# --- attention ----------------------------------------------------------------

import synth  # noqa: E402


def _fp16_cases():
    """Every rounding boundary of binary32 -> binary16: for each sign and binary32
    exponent, every pattern of the significand bits that survive, with the dropped
    bits at 0, 1, just below, at and just above the half-way point, and all ones;
    plus 4M random bit patterns."""
    out = [np.random.default_rng(61).integers(0, 1 << 32, 1 << 22, dtype=np.uint64).astype(np.uint32)]
    for e in range(256):
        ue = e - 127
        shift = 13 if ue >= -14 else min(24, -1 - ue)
        shift = min(shift, 23)
        half = 1 << (shift - 1)
        lows = np.array(sorted({0, 1, half - 1, half, half + 1, (1 << shift) - 1}), np.uint32)
        highs = np.arange(1 << (23 - shift), dtype=np.uint32) << np.uint32(shift)
        mant = (highs[:, None] | lows[None, :]).ravel()
        for sign in (0, 1):
            out.append((np.uint32(sign << 31) | np.uint32(e << 23) | mant).astype(np.uint32))
    return np.concatenate(out)


def test_f32_to_fp16_rounding_boundaries_against_numpy():
    bits = _fp16_cases()
    x = bits.view(np.float32)
    with np.errstate(over="ignore", invalid="ignore"):
        ref = x.astype(np.float16).view(np.uint16)
    got = oracle.f32_to_fp16_bits(x)
    nan = np.isnan(x)
    bad = np.nonzero(got[~nan] != ref[~nan])[0]
    assert bad.size == 0, [hex(int(v)) for v in bits[~nan][bad[:5]]]
    assert np.all((got[nan] & 0x7c00) == 0x7c00) and np.all(got[nan] & 0x3ff)


def test_rope_pair_special_angles_and_complex_rotation():
    assert oracle.rope_pair(1.5, -2.25, 1.0, 0.0) == (1.5, -2.25)        # angle 0
    assert oracle.rope_pair(1.5, -2.25, 0.0, 1.0) == (2.25, 1.5)         # a quarter turn
    assert oracle.rope_pair(1.5, -2.25, -1.0, 0.0) == (-1.5, 2.25)       # a half turn
    rng = np.random.default_rng(21)
    for mode, pair in ((oracle.ROPE_NORM, lambda i: (2 * i, 2 * i + 1)),
                       (oracle.ROPE_NEOX, lambda i: (i, i + 64))):
        L, D, nh = 37, 128, 3
        tab = synth.rope_table(L, D, 10000.0)
        x = rng.standard_normal((L, nh * D)).astype(np.float32)
        y = oracle.rope_rows(x, nh, D, tab, mode)
        for h in range(nh):
            for i in range(D // 2):
                a, b = pair(i)
                z = (x[:, h * D + a].astype(np.float64) + 1j * x[:, h * D + b]) * \
                    (tab[:, i, 0].astype(np.float64) + 1j * tab[:, i, 1])
                mag = np.abs(z) + 1e-30
                assert np.all(np.abs(y[:, h * D + a] - z.real) <= 4e-7 * mag)
                assert np.all(np.abs(y[:, h * D + b] - z.imag) <= 4e-7 * mag)


def _f16(x):
    return np.asarray(x, np.float32).astype(np.float16).astype(np.float64)


def test_attention_closed_forms():
    rng = np.random.default_rng(31)
    H, Hkv, D = 4, 2, 128
    # one position: the output is its own value vector
    qkv = synth.qkv_rows(rng, 1, H, Hkv, D)
    out, _ = oracle.attention(qkv, H, Hkv, D)
    v = _f16(qkv[0, (H + Hkv) * D:])
    for h in range(H):
        assert np.array_equal(out[0, h * D:(h + 1) * D], v[(h // 2) * D:(h // 2 + 1) * D])
    # equal keys: uniform weights, the mean of the values
    L = 9
    qkv = synth.qkv_rows(rng, L, H, Hkv, D)
    qkv[:, H * D:(H + Hkv) * D] = qkv[0, H * D:(H + Hkv) * D]
    out, tol = oracle.attention(qkv, H, Hkv, D)
    vmean = _f16(qkv[:, (H + Hkv) * D:]).mean(axis=0)
    for h in range(H):
        g = h // 2
        np.testing.assert_allclose(out[:, h * D:(h + 1) * D],
                                   np.broadcast_to(vmean[g * D:(g + 1) * D], (L, D)),
                                   rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(tol[:, :D], np.broadcast_to(np.abs(_f16(qkv[:, (H + Hkv) * D:
                                                                       (H + Hkv) * D + D])).mean(0), (L, D)),
                               rtol=1e-12)
    # constant values: the output is that constant, whatever the weights
    qkv = synth.qkv_rows(rng, L, H, Hkv, D, scale=2.0)
    qkv[:, (H + Hkv) * D:] = qkv[3, (H + Hkv) * D:]
    out, _ = oracle.attention(qkv, H, Hkv, D)
    v = _f16(qkv[3, (H + Hkv) * D:])
    for h in range(H):
        np.testing.assert_allclose(out[:, h * D:(h + 1) * D],
                                   np.broadcast_to(v[(h // 2) * D:(h // 2 + 1) * D], (L, D)),
                                   rtol=1e-13)


def test_attention_two_keys():
    # one head, D = 2: q = (1, 0); keys (a, 0) and (b, 0); values (1, 0) and (0, 1):
    # the output is (p, 1 - p) with p = 1 / (1 + exp((b - a) / sqrt(2)))
    H, Hkv, D = 1, 1, 2
    a, b = 3.0, 1.0
    qkv = np.array([[1, 0, a, 0, 1, 0],
                    [0.5, 0.25, b, 0, 0, 1]], np.float32)
    out, _ = oracle.attention(qkv, H, Hkv, D)
    p = 1.0 / (1.0 + np.exp((b - a) / np.sqrt(2.0)))
    np.testing.assert_allclose(out[0], [p, 1 - p], rtol=1e-14)
    # position 1's query (0.5, 0.25): scores 0.5 a and 0.5 b
    p1 = 1.0 / (1.0 + np.exp(0.5 * (b - a) / np.sqrt(2.0)))
    np.testing.assert_allclose(out[1], [p1, 1 - p1], rtol=1e-14)


def test_attention_permutation_and_shared_kv_heads():
    rng = np.random.default_rng(41)
    L, H, Hkv, D = 23, 6, 2, 128
    qkv = synth.qkv_rows(rng, L, H, Hkv, D, scale=1.5)
    out, _ = oracle.attention(qkv, H, Hkv, D)
    perm = rng.permutation(L)
    outp, _ = oracle.attention(qkv[perm], H, Hkv, D)
    np.testing.assert_allclose(outp, out[perm], rtol=1e-12, atol=1e-14)
    # heads 0 and 2 share kv head 0 (groups of 3): equal queries give equal outputs
    qkv2 = qkv.copy()
    qkv2[:, 2 * D:3 * D] = qkv2[:, 0:D]
    out2, _ = oracle.attention(qkv2, H, Hkv, D)
    assert np.array_equal(out2[:, 0:D], out2[:, 2 * D:3 * D])
    assert not np.array_equal(out2[:, 0:D], out2[:, 3 * D:4 * D])  # head 3 reads kv head 1


@pytest.mark.parametrize("mode", [1, 2])
def test_attention_rope_scores_depend_on_relative_position(mode):
    # every position's q and k equal: with RoPE, position i's scores over the keys j
    # depend on i - j only, so position i attends to a shifted copy of the pattern of
    # position 0 (checked on the weights, through one-hot values)
    rng = np.random.default_rng(51)
    L, D = 8, 128
    qk = rng.standard_normal(D).astype(np.float32)
    tab = synth.rope_table(L, D, 10000.0)
    qkv = np.zeros((L, 3 * D + 0), np.float32)
    # values: position j carries the unit vector e_j in its first L dims
    qkv[:, 0:D] = qk
    qkv[:, D:2 * D] = qk
    qkv[np.arange(L), 2 * D + np.arange(L)] = 1.0
    out, _ = oracle.attention(qkv, 1, 1, D, tab, mode)
    w = out[:, :L]  # w[i, j] = attention weight of position i on key j
    np.testing.assert_allclose(w.sum(axis=1), 1.0, rtol=1e-12)
    # scores s(i, j) = f(i - j): w[i, j] / w[i, j'] = w[0, j - i] / w[0, j' - i] where in range
    for i in range(1, L):
        for j in range(i, L):
            r1 = np.log(w[i, j]) - np.log(w[i, i])
            r0 = np.log(w[0, j - i]) - np.log(w[0, 0])
            assert abs(r1 - r0) < 0.05, (i, j, r1, r0)  # binary16 rounding of rotated vectors
    # without RoPE every score is the same: uniform weights
    out0, _ = oracle.attention(qkv, 1, 1, D)
    np.testing.assert_allclose(out0[:, :L], 1.0 / L, rtol=1e-12)


# --- the decoder's other block types --------------------------------------------

from kq_fields import (dequant_q5k_fields, dequant_q8_0_fields, enc_q5k, enc_q8_0,  # noqa: E402
                       encode_q5k_matrix, encode_q8_0_matrix, random_q5k_fields,
                       random_q8_0_fields)


def test_f16_and_bf16_rows():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    w = oracle.decode_row(oracle.F16, bits.view(np.uint8), 1 << 16)
    ref = bits.view(np.float16).astype(np.float64)
    fin = np.isfinite(ref)
    assert np.array_equal(w[fin], ref[fin])
    assert np.all(np.isinf(w[np.isinf(ref)])) and np.all(np.isnan(w[np.isnan(ref)]))
    consts = {0x3F80: 1.0, 0xC000: -2.0, 0x3E20: 0.15625, 0x4049: 3.140625, 0x0000: 0.0,
              0x0001: 2.0 ** -133, 0x7F7F: 3.3895313892515355e38}
    keys = np.array(list(consts), np.uint16)
    w = oracle.decode_row(oracle.BF16, keys.view(np.uint8), len(keys))
    assert np.array_equal(w, np.array(list(consts.values())))
    # every binary32 with a zero low half is its own top half
    x = (np.random.default_rng(71).integers(0, 1 << 16, 4096).astype(np.uint32) << 16)
    x = x[np.isfinite(x.view(np.float32))]
    w = oracle.decode_row(oracle.BF16, (x >> 16).astype(np.uint16).view(np.uint8), x.size)
    assert np.array_equal(w, x.view(np.float32).astype(np.float64))
    f = np.random.default_rng(72).standard_normal(300).astype(np.float32)
    assert np.array_equal(oracle.decode_row(oracle.F32, f.view(np.uint8), 300), f.astype(np.float64))


def test_q8_0_closed_form_and_round_trip():
    q = np.arange(-128, 128, dtype=np.int64).reshape(8, 32)
    row = np.concatenate([enc_q8_0(0.5, q[b]) for b in range(8)])
    d, qq = oracle.decode_q8_0(row[:34])
    assert d == 0.5 and np.array_equal(qq, q[0])
    assert np.array_equal(oracle.decode_row(oracle.Q8_0, row, 256), np.arange(-128, 128) / 2.0)
    f = random_q8_0_fields(np.random.default_rng(73), 5, 6)
    W = encode_q8_0_matrix(f).reshape(5, -1)
    for n in range(5):
        assert np.array_equal(oracle.decode_row(oracle.Q8_0, W[n], 192), dequant_q8_0_fields(f)[n])


def test_q5k_closed_form_and_round_trip():
    # d = 1, dmin = 0.5, sc_j = j + 1 (the high-bit scales need j >= 4 slots up to 63),
    # m_j = 2j, q_i = i mod 32 (the fifth bit set in half of each chunk)
    sc = [1, 2, 3, 4, 61, 62, 63, 40]
    mn = [0, 2, 4, 6, 8, 63, 12, 14]
    q = np.arange(256) % 32
    blk = enc_q5k(1.0, 0.5, sc, mn, q)
    d, dm, s2, m2, q2 = oracle.decode_q5k(blk)
    assert (d, dm) == (1.0, 0.5)
    assert list(s2) == sc and list(m2) == mn and np.array_equal(q2, q)
    ref = np.array([sc[i // 32] * q[i] - 0.5 * mn[i // 32] for i in range(256)], np.float64)
    assert np.array_equal(oracle.decode_row(oracle.Q5_K, blk, 256), ref)
    f = random_q5k_fields(np.random.default_rng(74), 4, 3)
    W = encode_q5k_matrix(f).reshape(4, -1)
    for n in range(4):
        assert np.array_equal(oracle.decode_row(oracle.Q5_K, W[n], 768), dequant_q5k_fields(f)[n])


def test_embed_rows_select_and_flag():
    rng = np.random.default_rng(75)
    N, K = 7, 512
    f = random_q5k_fields(rng, N, K // 256)
    table = encode_q5k_matrix(f).reshape(N, -1)
    ids = np.array([3, 0, 6, 3, -1, 7], np.int32)
    out, flag = oracle.embed_rows(oracle.Q5_K, table, K, ids)
    ref = dequant_q5k_fields(f).astype(np.float32)
    assert np.array_equal(flag, [0, 0, 0, 0, 1, 1])
    assert np.array_equal(out[:4], ref[ids[:4]]) and not out[4:].any()
    assert oracle.row_bytes(oracle.Q8_0, 100) == 0 and oracle.row_bytes(99, 256) == 0
