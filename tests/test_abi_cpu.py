"""The C-ABI library on the CPU: it loads, exports every symbol include/dq.h
declares, and its host-side checks return the documented status codes (none of
these calls reaches a kernel launch)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dq.h")

dq = pytest.importorskip("quantized_gemm_diffusion_amd")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(dq.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    return dq.load_library()


def declared_symbols():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(dq_\w+)\s*\(", text, re.M)))


def test_exports_every_declared_symbol(lib):
    syms = declared_symbols()
    assert len(syms) >= 9
    assert sorted(dq.EXPORTS) == syms
    for s in syms:
        assert hasattr(lib, s), s


def _doc_blocks():
    """The comment block in front of each declaration of include/dq.h."""
    text = open(HEADER).read()
    blocks = {}
    for m in re.finditer(r"/\*(.*?)\*/\s*(?:#define[^\n]*\n\s*)?((?:int|const char \*)[^;]*;\s*)+",
                         text, re.S):
        for name in re.findall(r"(dq_\w+)\s*\(", m.group(0)[m.group(0).rfind("*/"):]):
            blocks[name] = m.group(1)
    return blocks


def test_every_entry_point_cites_its_source():
    # each declaration's comment names the passage it implements (the size
    # queries among them); the allocation-free variant names its callers instead
    blocks = _doc_blocks()
    for name in declared_symbols():
        if name in ("dq_status_string", "dq_last_error"):
            continue
        doc = blocks.get(name)
        assert doc is not None, name
        if name == "dq_qgemm_rows_noalloc":
            assert "cannot allocate" in doc, name
        else:
            flat = re.sub(r"\s*\n\s*\*\s*", " ", doc)  # the comment as one line
            assert "Source" in flat or "as for dq_" in flat or "Runs the dq_qgemm kernel" in flat, name
    for q in ("dq_packed_size", "dq_act_size", "dq_qgemm_rows_workspace"):
        assert "Source" in blocks[q], q


def test_status_strings(lib):
    assert lib.dq_status_string(dq.DQ_OK) == b"DQ_OK"
    assert lib.dq_status_string(dq.DQ_EWORKSPACE) == b"DQ_EWORKSPACE"
    assert lib.dq_status_string(99) == b"DQ_UNKNOWN"


@pytest.mark.parametrize("type_,N,K,exp", [
    (dq.Q4_K, 4096, 4096, 4096 * 16 * 144),
    (dq.Q6_K, 126464, 4096, 126464 * 16 * 210),
    (dq.Q4_K, 33, 512, 48 * 2 * 144),      # rounded up to 16-row tiles
    (dq.Q6_K, 1, 256, 16 * 210),
    (dq.Q4_K, 0, 256, 0),
])
def test_packed_size(lib, type_, N, K, exp):
    assert dq.packed_size(type_, N, K) == exp


def _status(fn, *args):
    return fn(*args)


def test_host_checks_return_codes(lib):
    out = ctypes.c_size_t()
    assert lib.dq_packed_size(13, 32, 256, ctypes.byref(out)) == dq.DQ_EUNSUPPORTED
    assert lib.dq_packed_size(dq.Q4_K, 32, 300, ctypes.byref(out)) == dq.DQ_EINVAL
    assert b"multiple of 256" in lib.dq_last_error()
    assert lib.dq_packed_size(dq.Q4_K, -1, 256, ctypes.byref(out)) == dq.DQ_EINVAL
    assert lib.dq_packed_size(dq.Q4_K, 32, 256, None) == dq.DQ_EINVAL
    # NULL device pointers are refused before any launch
    assert lib.dq_qgemm(dq.Q4_K, 4, 32, 256, None, None, None, 32, None) == dq.DQ_EINVAL
    assert lib.dq_qgemm(15, 4, 32, 256, None, None, None, 32, None) == dq.DQ_EUNSUPPORTED
    assert lib.dq_qgemm(dq.Q4_K, 4, 32, 512, 16, 16, 16, 31, None) == dq.DQ_EINVAL  # ldy < N
    assert lib.dq_qgemm(dq.Q4_K, 4, 32, 512, 8, 16, 16, 32, None) == dq.DQ_EINVAL  # qa misaligned
    assert lib.dq_qgemm(dq.Q4_K, 4, 32, 512, 16, 16, None, 32, None) == dq.DQ_EINVAL  # y NULL
    assert lib.dq_quantize_act(4, 512, 16, 500, 16, None) == dq.DQ_EINVAL  # ldx < K
    assert lib.dq_quantize_act(4, 100, 16, 100, 16, None) == dq.DQ_EINVAL
    assert lib.dq_quantize_act(4, 512, 16, 512, 8, None) == dq.DQ_EINVAL  # qa misaligned
    assert lib.dq_repack_weights(dq.Q6_K, 32, 256, None, 16, None) == dq.DQ_EINVAL
    assert lib.dq_repack_weights(dq.Q6_K, 32, 256, 16, 8, None) == dq.DQ_EINVAL  # packed misaligned
    assert lib.dq_act_size(1 << 20, 1 << 14, ctypes.byref(out)) == dq.DQ_EINVAL  # > 2^31 bytes
    # the fused producers
    assert lib.dq_swiglu_quantize_act(4, 512, 16, 1000, 16, None) == dq.DQ_EINVAL  # ldgu < 2F
    assert lib.dq_swiglu_quantize_act(4, 300, 16, 600, 16, None) == dq.DQ_EINVAL  # F % 256
    assert lib.dq_swiglu_quantize_act(4, 512, None, 1024, 16, None) == dq.DQ_EINVAL
    assert lib.dq_swiglu_quantize_act(4, 512, 16, 1024, 8, None) == dq.DQ_EINVAL  # qa misaligned
    assert lib.dq_rmsnorm_quantize_act(4, 512, 16, 500, 16, 1e-5, 16, None) == dq.DQ_EINVAL
    assert lib.dq_rmsnorm_quantize_act(4, 512, 16, 512, 16, -1.0, 16, None) == dq.DQ_EINVAL
    assert lib.dq_rmsnorm_quantize_act(4, 512, 16, 512, 16, float("nan"), 16, None) == dq.DQ_EINVAL
    assert lib.dq_rmsnorm_quantize_act(4, 512, 16, 512, None, 1e-5, 16, None) == dq.DQ_EINVAL
    assert lib.dq_rmsnorm_quantize_act(4, 512, 16, 512, 16, 1e-5, 8, None) == dq.DQ_EINVAL
    # one sum of squares per 256-block in LDS: K at most 262144
    assert lib.dq_rmsnorm_quantize_act(1, 262400, 16, 262400, 16, 1e-5, 16, None) == dq.DQ_EINVAL
    # empty shapes are valid no-ops
    assert lib.dq_qgemm(dq.Q4_K, 0, 32, 256, None, None, None, 32, None) == dq.DQ_OK
    # the gate/up GEMM with SiLU(gate) * up in its epilogue
    assert lib.dq_qgemm_swiglu(dq.Q4_K, 4, 24, 512, 16, 16, 16, 24, None) == dq.DQ_EINVAL  # F % 16
    assert lib.dq_qgemm_swiglu(dq.Q4_K, 4, 32, 512, 16, 16, 16, 31, None) == dq.DQ_EINVAL  # ldh < F
    assert lib.dq_qgemm_swiglu(dq.Q4_K, 4, 32, 512, 16, 16, None, 32, None) == dq.DQ_EINVAL  # h NULL
    assert lib.dq_qgemm_swiglu(dq.Q4_K, 4, 32, 512, 8, 16, 16, 32, None) == dq.DQ_EINVAL  # qa misaligned
    assert lib.dq_qgemm_swiglu(15, 4, 32, 512, 16, 16, 16, 32, None) == dq.DQ_EUNSUPPORTED
    assert lib.dq_qgemm_swiglu(dq.Q4_K, 0, 32, 256, None, None, None, 32, None) == dq.DQ_OK
    assert lib.dq_qgemm_swiglu(dq.Q4_K, 4, 0, 256, None, None, None, 0, None) == dq.DQ_OK
    assert lib.dq_quantize_act(0, 256, None, 256, None, None) == dq.DQ_OK
    assert lib.dq_swiglu_quantize_act(0, 256, None, 512, None, None) == dq.DQ_OK
    assert lib.dq_rmsnorm_quantize_act(0, 256, None, 256, None, 0.0, None, None) == dq.DQ_OK


@pytest.mark.parametrize("M,K,exp", [
    (160, 4096, 10 * 16 * 5120),
    (1, 256, 5120),
    (17, 512, 2 * 2 * 5120),     # rows rounded up to blocks of 16
    (0, 256, 0),
])
def test_act_size(lib, M, K, exp):
    assert dq.act_size(M, K) == exp


def test_rows_workspace(lib):
    need = dq.qgemm_rows_workspace(32, 4096)
    assert need == 256 + dq.act_size(32, 4096)  # flags, then the activation records
    # short workspace -> DQ_EWORKSPACE, before anything is launched
    st = lib.dq_qgemm_rows(dq.Q6_K, 160, 32, 126464, 4096, 256, 4096, 256, 256, 256, 126464,
                           256, need - 1, None)
    assert st == dq.DQ_EWORKSPACE
    st = lib.dq_qgemm_rows(dq.Q6_K, 160, 32, 126464, 4096, 256, 4096, 256, 256, 256, 126464,
                           None, need, None)
    assert st == dq.DQ_EWORKSPACE
    assert lib.dq_qgemm_rows_workspace(4, 100, None) == dq.DQ_EINVAL


def test_sampler_workspaces_and_host_checks(lib):
    # standalone: one 16-byte state per 4096 columns per row
    assert dq.logits_stats_workspace(32, 126464) == 32 * 31 * 16
    assert dq.logits_stats_workspace(3, 1) == 3 * 16
    # fused: the narrow kernel (M <= 32, K/256 even in [8, 16], >= 1024 n-tiles) keeps one
    # state per row per workgroup (256), the canvas kernel one per 32-column group
    rows = dq.qgemm_rows_workspace(32, 4096)
    assert dq.qgemm_rows_sample_workspace(32, 126464, 4096) == rows + 32 * 256 * 16
    assert dq.qgemm_rows_sample_workspace(64, 152064, 3584) == \
        dq.qgemm_rows_workspace(64, 3584) + 64 * 4752 * 16
    assert dq.qgemm_rows_sample_workspace(8, 4096, 4096) == \
        dq.qgemm_rows_workspace(8, 4096) + 8 * 128 * 16
    out = ctypes.c_size_t()
    assert lib.dq_logits_stats_workspace(4, 0, ctypes.byref(out)) == dq.DQ_EINVAL
    assert lib.dq_qgemm_rows_sample_workspace(4, 0, 256, ctypes.byref(out)) == dq.DQ_EINVAL
    assert lib.dq_qgemm_rows_sample_workspace(4, 256, 100, ctypes.byref(out)) == dq.DQ_EINVAL
    need = dq.logits_stats_workspace(4, 1000)
    for beta in (0.0, -1.0, float("nan"), float("inf")):
        assert lib.dq_logits_stats(4, 1000, 16, 1000, beta, 16, 16, 256, need, None) == dq.DQ_EINVAL
        assert lib.dq_qgemm_rows_sample(dq.Q6_K, 160, 4, 4096, 4096, 256, 4096, 256, 256, beta,
                                        16, 16, 256, 1 << 30, None) == dq.DQ_EINVAL
    assert lib.dq_logits_stats(4, 1000, 16, 999, 1.0, 16, 16, 256, need, None) == dq.DQ_EINVAL
    assert lib.dq_logits_stats(4, 1000, None, 1000, 1.0, 16, 16, 256, need, None) == dq.DQ_EINVAL
    assert lib.dq_logits_stats(4, 1000, 16, 1000, 1.0, 16, 16, 256, need - 1, None) == \
        dq.DQ_EWORKSPACE
    assert lib.dq_logits_stats(4, 1000, 16, 1000, 1.0, 16, 16, 8, need, None) == dq.DQ_EINVAL
    ws = dq.qgemm_rows_sample_workspace(32, 126464, 4096)
    assert lib.dq_qgemm_rows_sample(dq.Q6_K, 160, 32, 126464, 4096, 256, 4096, 256, 256, 1.0,
                                    16, 16, 256, ws - 1, None) == dq.DQ_EWORKSPACE
    assert lib.dq_qgemm_rows_sample(dq.Q6_K, 160, 32, 126464, 4096, 256, 4096, 256, 256, 1.0,
                                    16, None, 256, ws, None) == dq.DQ_EINVAL
    assert lib.dq_qgemm_rows_sample(7, 160, 32, 126464, 4096, 256, 4096, 256, 256, 1.0,
                                    16, 16, 256, ws, None) == dq.DQ_EUNSUPPORTED
    # empty row lists are valid no-ops
    assert lib.dq_logits_stats(0, 1000, None, 1000, 1.0, None, None, None, 0, None) == dq.DQ_OK
    assert lib.dq_qgemm_rows_sample(dq.Q6_K, 160, 0, 4096, 4096, None, 4096, None, None, 1.0,
                                    None, None, None, 0, None) == dq.DQ_OK


def test_attention_host_checks(lib):
    ld = (32 + 2 * 32) * 128
    need = dq.attention_workspace(160, 32, 32)
    assert need == 32 * 5 * 20480                    # per kv head and 32 keys, one 20 KB image
    assert dq.attention_workspace(512, 28, 4) == 4 * 16 * 20480
    ok_args = dict(L=160, H=32, Hkv=32, D=128, qkv=256, ldqkv=ld, rope=256, mode=1, out=256,
                   ldo=4096, ws=256, wsb=need)

    def call(**kw):
        a = dict(ok_args, **kw)
        return lib.dq_attention(a["L"], a["H"], a["Hkv"], a["D"], a["qkv"], a["ldqkv"], a["rope"],
                                a["mode"], a["out"], a["ldo"], a["ws"], a["wsb"], None)
    assert call(D=64) == dq.DQ_EUNSUPPORTED
    assert call(Hkv=5) == dq.DQ_EINVAL              # does not divide H
    assert call(Hkv=0) == dq.DQ_EINVAL
    assert call(mode=3) == dq.DQ_EINVAL
    assert call(ldqkv=ld - 4) == dq.DQ_EINVAL        # shorter than the three blocks
    assert call(ldqkv=ld + 2) == dq.DQ_EINVAL        # not a multiple of 4
    assert call(ldo=4095) == dq.DQ_EINVAL
    assert call(qkv=None) == dq.DQ_EINVAL
    assert call(rope=None) == dq.DQ_EINVAL           # NORM needs the table
    assert call(qkv=264) == dq.DQ_EINVAL             # qkv not 16-byte aligned
    assert call(rope=260) == dq.DQ_EINVAL            # rope not 8-byte aligned
    assert call(wsb=need - 1) == dq.DQ_EWORKSPACE
    assert call(ws=None) == dq.DQ_EWORKSPACE
    assert call(ws=264) == dq.DQ_EINVAL              # workspace not 16-byte aligned
    assert call(L=0) == dq.DQ_OK                     # empty canvas: nothing to do


def test_embed_rows_host_checks(lib):
    for t, K, b in ((0, 512, 2048), (1, 512, 1024), (30, 512, 1024), (8, 512, 544),
                    (12, 4096, 2304), (13, 4096, 2816), (14, 4096, 3360)):
        assert dq.row_bytes(t, K) == b
    out = ctypes.c_size_t()
    assert lib.dq_row_bytes(2, 256, ctypes.byref(out)) == dq.DQ_EUNSUPPORTED   # Q4_0: not decoded
    assert lib.dq_row_bytes(8, 288, ctypes.byref(out)) == dq.DQ_EINVAL        # not 256-aligned
    assert lib.dq_embed_rows(12, 10, 4096, 256, 256, 4, 256, 4095, None, None) == dq.DQ_EINVAL
    assert lib.dq_embed_rows(12, 10, 4096, 264, 256, 4, 256, 4096, None, None) == dq.DQ_EINVAL
    assert lib.dq_embed_rows(12, 10, 4096, None, 256, 4, 256, 4096, None, None) == dq.DQ_EINVAL
    assert lib.dq_embed_rows(12, 10, 4096, None, None, 0, None, 4096, None, None) == dq.DQ_OK
