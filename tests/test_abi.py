"""The C-ABI library loads, exports every declared symbol, and rejects bad
arguments on the host before any HIP call (CPU only: nothing is launched)."""
import ctypes
import os
import re
import subprocess

import pytest

import tiled_attention_16_amd as ta

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "tiled_attention_16_amd", "libattn.so")


def declared_functions():
    text = open(os.path.join(ROOT, "include", "attn.h"), encoding="utf-8").read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(attn_\w+)\s*\(", text, flags=re.M)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        pytest.fail("libattn.so is not built: run __graft_entry__.build()")
    return ta.load_library()


def test_header_declares_the_entry_points():
    assert declared_functions() == sorted(ta.EXPORTS)


def test_every_declared_symbol_is_exported(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", LIB], capture_output=True, text=True, check=True).stdout
    exported = set(re.findall(r"\sT\s(\w+)$", out, flags=re.M))
    for name in declared_functions():
        assert name in exported, name
        assert getattr(lib, name) is not None


def test_version_and_status_strings(lib):
    assert ta.attn_version() == 10100
    for code in range(10):
        s = ta.attn_status_str(code)
        assert s and s != "unknown status"
    assert ta.attn_status_str(99) == "unknown status"


A16 = 0x10000   # a 16-byte aligned fake address: never dereferenced, the call returns first


def call(**kw):
    args = dict(q=A16, k=A16 * 2, v=A16 * 3, o=A16 * 4, lse=A16 * 5, B=1, H=2, N_q=8, N_k=8, d=64, scale=0.125,
                causal=False, seqlens_k=0, q_start=0, stream=0)
    args.update(kw)
    return ta.attn_fwd_raw(**args)


@pytest.mark.parametrize("kw,status", [
    (dict(B=-1), ta.ATTN_ERR_SHAPE),
    (dict(N_k=-3), ta.ATTN_ERR_SHAPE),
    (dict(d=96), ta.ATTN_ERR_HEAD_DIM),
    (dict(d=0), ta.ATTN_ERR_HEAD_DIM),
    (dict(scale=float("nan")), ta.ATTN_ERR_SCALE),
    (dict(scale=float("inf")), ta.ATTN_ERR_SCALE),
    (dict(q=0), ta.ATTN_ERR_NULL),
    (dict(o=0), ta.ATTN_ERR_NULL),
    (dict(k=0), ta.ATTN_ERR_NULL),
    (dict(q=A16 + 8), ta.ATTN_ERR_ALIGN),
    (dict(v=A16 * 3 + 2), ta.ATTN_ERR_ALIGN),
    (dict(lse=A16 * 5 + 2), ta.ATTN_ERR_ALIGN),
    (dict(o=A16 + 16), ta.ATTN_ERR_ALIAS),          # o overlaps q (2*8*64*2 bytes long)
    (dict(lse=A16 * 4 + 64), ta.ATTN_ERR_ALIAS),    # lse inside o
    (dict(B=1 << 20, H=1 << 12, N_q=1 << 12), ta.ATTN_ERR_SHAPE),   # too many workgroups
    (dict(N_k=1 << 23, d=128), ta.ATTN_ERR_SHAPE),   # one head's K spans 2 GB
    (dict(causal=3), ta.ATTN_ERR_MASK),
    (dict(causal=-1), ta.ATTN_ERR_MASK),
])
def test_argument_errors_return_before_any_hip_call(lib, kw, status):
    assert call(**kw) == status


def test_empty_problem_is_a_noop(lib):
    # nothing to write: returns OK without touching the (NULL) pointers or the GPU
    assert call(B=0, q=0, o=0, lse=0) == ta.ATTN_OK
    assert call(N_q=0, q=0, o=0, lse=0, k=0, v=0) == ta.ATTN_OK


def test_binding_rejects_cpu_tensors(lib):
    torch = pytest.importorskip("torch")
    q = torch.zeros(1, 1, 4, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        ta.attn_fwd(q, q, q)


def test_missing_library_fails_loudly(monkeypatch):
    monkeypatch.setattr(ta, "_lib", None)
    monkeypatch.setattr(ta, "_LIB_PATH", "/nonexistent/libattn.so")
    with pytest.raises(RuntimeError):
        ta.load_library()


def call_bwd(**kw):
    args = dict(q=A16, k=A16 * 2, v=A16 * 3, o=A16 * 4, dout=A16 * 5, lse=A16 * 6, dq=A16 * 7, dk=A16 * 8,
                dv=A16 * 9, delta=A16 * 10, B=1, H=2, N_q=8, N_k=8, d=64, scale=0.125, causal=False, seqlens_k=0,
                q_start=0, stream=0)
    args.update(kw)
    return ta.attn_bwd_raw(**args)


@pytest.mark.parametrize("kw,status", [
    (dict(H=-1), ta.ATTN_ERR_SHAPE),
    (dict(d=32), ta.ATTN_ERR_HEAD_DIM),
    (dict(scale=float("-inf")), ta.ATTN_ERR_SCALE),
    (dict(dout=0), ta.ATTN_ERR_NULL),
    (dict(lse=0), ta.ATTN_ERR_NULL),
    (dict(delta=0), ta.ATTN_ERR_NULL),
    (dict(dk=0), ta.ATTN_ERR_NULL),
    (dict(dq=A16 * 7 + 8), ta.ATTN_ERR_ALIGN),
    (dict(dout=A16 * 5 + 4), ta.ATTN_ERR_ALIGN),
    (dict(delta=A16 * 10 + 2), ta.ATTN_ERR_ALIGN),
    (dict(dq=A16 * 5 + 16), ta.ATTN_ERR_ALIAS),       # dq overlaps dout
    (dict(dv=A16 * 8 + 32), ta.ATTN_ERR_ALIAS),       # dv overlaps dk
    (dict(delta=A16 * 6), ta.ATTN_ERR_ALIAS),         # delta is lse
    (dict(causal=7), ta.ATTN_ERR_MASK),
])
def test_bwd_argument_errors_return_before_any_hip_call(lib, kw, status):
    assert call_bwd(**kw) == status


def test_bwd_empty_problem_is_a_noop(lib):
    assert call_bwd(B=0, q=0, k=0, v=0, o=0, dout=0, lse=0, dq=0, dk=0, dv=0, delta=0) == ta.ATTN_OK
    assert call_bwd(N_q=0, N_k=0, q=0, k=0, v=0, o=0, dout=0, lse=0, dq=0, dk=0, dv=0, delta=0) == ta.ATTN_OK


def test_causal_mode_names():
    assert [ta.causal_mode(x) for x in (False, True, "none", "top_left", "bottom_right", 2)] == [0, 1, 0, 1, 2, 2]
    with pytest.raises(ValueError):
        ta.causal_mode("diagonal")


def call_masked(**kw):
    args = dict(q=A16, k=A16 * 2, v=A16 * 3, o=A16 * 4, lse=A16 * 5, B=1, H=2, N_q=8, N_k=300, d=64, scale=0.125,
                causal=False, seqlens_k=0, q_start=0, mask_bits=A16 * 40, mask_stride_b=0, mask_stride_h=0,
                mask_row_words=16, stream=0)
    args.update(kw)
    return ta.attn_fwd_masked_raw(**args)


@pytest.mark.parametrize("kw,status", [
    (dict(mask_bits=0), ta.ATTN_ERR_NULL),
    (dict(mask_bits=A16 * 40 + 4), ta.ATTN_ERR_ALIGN),
    (dict(mask_row_words=8), ta.ATTN_ERR_MASK),          # 300 keys need 10 words
    (dict(mask_row_words=12), ta.ATTN_ERR_MASK),         # not a multiple of 8
    (dict(mask_stride_h=-1), ta.ATTN_ERR_MASK),
    (dict(causal=5), ta.ATTN_ERR_MASK),
    (dict(d=80), ta.ATTN_ERR_HEAD_DIM),
    (dict(N_q=1 << 22, mask_row_words=1 << 10), ta.ATTN_ERR_SHAPE),
])
def test_masked_argument_errors_return_before_any_hip_call(lib, kw, status):
    assert call_masked(**kw) == status


def test_mask_pack_argument_errors(lib):
    assert lib.attn_mask_pack(A16, A16 * 2, 4, 300, 9, None) == ta.ATTN_ERR_SHAPE    # 300 keys need 10 words
    assert lib.attn_mask_pack(A16, 0, 4, 300, 16, None) == ta.ATTN_ERR_NULL
    assert lib.attn_mask_pack(A16, A16 * 2 + 2, 4, 300, 16, None) == ta.ATTN_ERR_ALIGN
    assert lib.attn_mask_pack(0, 0, 0, 300, 16, None) == ta.ATTN_OK


def test_mask_row_words():
    assert [ta.mask_row_words(n) for n in (1, 256, 257, 4096)] == [8, 8, 16, 128]


def test_bwd_masked_argument_errors(lib):
    base = dict(q=A16, k=A16 * 2, v=A16 * 3, o=A16 * 4, dout=A16 * 5, lse=A16 * 6, dq=A16 * 7, dk=A16 * 8,
                dv=A16 * 9, delta=A16 * 10)
    p = [base[n] for n in ("q", "k", "v", "o", "dout", "lse", "dq", "dk", "dv", "delta")]
    common = p + [1, 2, 8, 300, 64, ctypes.c_float(0.125), 0, None, None]
    assert lib.attn_bwd_masked(*common, None, 0, 0, 16, None) == ta.ATTN_ERR_NULL
    assert lib.attn_bwd_masked(*common, A16 * 40 + 4, 0, 0, 16, None) == ta.ATTN_ERR_ALIGN
    assert lib.attn_bwd_masked(*common, A16 * 40, 0, 0, 8, None) == ta.ATTN_ERR_MASK
    assert lib.attn_bwd_masked(*common, A16 * 40, -1, 0, 16, None) == ta.ATTN_ERR_MASK


def test_block_sparse_argument_errors(lib):
    p = [A16, A16 * 2, A16 * 3, A16 * 4, A16 * 5, 1, 2, 8, 300, 64, ctypes.c_float(0.125), 0, None, None]
    assert lib.attn_fwd_block_sparse(*p, None, 0, 0, None) == ta.ATTN_ERR_NULL
    assert lib.attn_fwd_block_sparse(*p, A16 * 40, -1, 0, None) == ta.ATTN_ERR_MASK
    p_long = p[:8] + [40000] + p[9:]
    assert lib.attn_fwd_block_sparse(*p_long, A16 * 40, 0, 0, None) == ta.ATTN_ERR_SHAPE   # > 32768 keys
    p_bad = p[:11] + [3] + p[12:]
    assert lib.attn_fwd_block_sparse(*p_bad, A16 * 40, 0, 0, None) == ta.ATTN_ERR_MASK


def test_bwd_block_sparse_argument_errors(lib):
    p = [A16, A16 * 2, A16 * 3, A16 * 4, A16 * 5, A16 * 6, A16 * 7, A16 * 8, A16 * 9, A16 * 10, 1, 2, 8, 300, 64,
         ctypes.c_float(0.125), 0, None, None]
    assert lib.attn_bwd_block_sparse(*p, None, 0, 0, None) == ta.ATTN_ERR_NULL
    assert lib.attn_bwd_block_sparse(*p, A16 * 40, 0, -2, None) == ta.ATTN_ERR_MASK
    p_long = p[:12] + [40000] + p[13:]
    assert lib.attn_bwd_block_sparse(*p_long, A16 * 40, 0, 0, None) == ta.ATTN_ERR_SHAPE


def call_fp8(**kw):
    args = dict(q=A16, k=A16 * 2, vt=A16 * 3, vt_row_stride=16, o=A16 * 4, lse=A16 * 5, B=1, H=2, N_q=8, N_k=8, d=64,
                scale=0.125, q_descale=0.01, k_descale=0.02, v_descale=0.03, causal=False, stream=0)
    args.update(kw)
    return ta.attn_fwd_fp8_raw(**args)


@pytest.mark.parametrize("kw,status", [
    (dict(B=-1), ta.ATTN_ERR_SHAPE),
    (dict(N_k=-1), ta.ATTN_ERR_SHAPE),
    (dict(d=32), ta.ATTN_ERR_HEAD_DIM),
    (dict(scale=float("nan")), ta.ATTN_ERR_SCALE),
    (dict(q_descale=float("inf")), ta.ATTN_ERR_SCALE),
    (dict(v_descale=float("nan")), ta.ATTN_ERR_SCALE),
    (dict(scale=1e30, q_descale=1e30), ta.ATTN_ERR_SCALE),   # the product overflows
    (dict(causal=3), ta.ATTN_ERR_MASK),
    (dict(q=0), ta.ATTN_ERR_NULL),
    (dict(vt=0), ta.ATTN_ERR_NULL),
    (dict(o=0), ta.ATTN_ERR_NULL),
    (dict(vt_row_stride=8), ta.ATTN_ERR_SHAPE),     # not a multiple of 16
    (dict(N_k=17, vt_row_stride=16), ta.ATTN_ERR_SHAPE),   # shorter than N_k rounded up to 16
    (dict(k=A16 * 2 + 4), ta.ATTN_ERR_ALIGN),
    (dict(lse=A16 * 5 + 1), ta.ATTN_ERR_ALIGN),
    (dict(o=A16 * 3), ta.ATTN_ERR_ALIAS),            # o on top of vt
    (dict(lse=A16 * 4 + 32), ta.ATTN_ERR_ALIAS),     # lse inside o
    (dict(B=1 << 20, H=1 << 12, N_q=1 << 12), ta.ATTN_ERR_SHAPE),
    (dict(N_k=1 << 25, vt_row_stride=1 << 25), ta.ATTN_ERR_SHAPE),   # a head's K/V^T past 32-bit load offsets
])
def test_fp8_argument_errors_return_before_any_hip_call(lib, kw, status):
    assert call_fp8(**kw) == status


def test_fp8_empty_problem_is_a_noop(lib):
    assert call_fp8(N_q=0, q=0, o=0, lse=0, k=0, vt=0) == ta.ATTN_OK
    assert call_fp8(B=0, q=0, o=0) == ta.ATTN_OK


def test_fp8_vt_stride():
    assert [ta.fp8_vt_stride(n) for n in (0, 1, 16, 17, 4096)] == [16, 16, 16, 32, 4096]


def test_fp8_binding_rejects_bad_tensors(lib):
    torch = pytest.importorskip("torch")
    q = torch.zeros(1, 1, 4, 64, dtype=torch.uint8)
    vt = torch.zeros(1, 1, 64, 16, dtype=torch.uint8)
    with pytest.raises(ValueError):   # CPU tensors
        ta.attn_fwd_fp8(q, q, vt, q_descale=1.0, k_descale=1.0, v_descale=1.0)
    with pytest.raises(ValueError):   # bf16 is not an FP8 code tensor
        ta.attn_fwd_fp8(q.to(torch.bfloat16), q, vt, q_descale=1.0, k_descale=1.0, v_descale=1.0)


def call_bwd_noalloc(**kw):
    args = dict(q=A16, k=A16 * 2, v=A16 * 3, o=A16 * 4, dout=A16 * 5, lse=A16 * 6, dq=A16 * 7, dk=A16 * 8,
                dv=A16 * 9, B=1, H=2, N_q=8, N_k=8, d=64, scale=0.125, causal=False, seqlens_k=0, q_start=0, stream=0)
    args.update(kw)
    return ta.attn_bwd_noalloc_raw(**args)


@pytest.mark.parametrize("kw,status", [
    (dict(H=-1), ta.ATTN_ERR_SHAPE),
    (dict(B=1, H=16, N_q=65537), ta.ATTN_ERR_SCRATCH),        # 1048592 rows > 2^20
    (dict(B=1024, H=1024, N_q=2), ta.ATTN_ERR_SCRATCH),
    (dict(d=32), ta.ATTN_ERR_HEAD_DIM),
    (dict(scale=float("nan")), ta.ATTN_ERR_SCALE),
    (dict(dout=0), ta.ATTN_ERR_NULL),
    (dict(lse=0), ta.ATTN_ERR_NULL),
    (dict(dq=A16 * 7 + 8), ta.ATTN_ERR_ALIGN),
    (dict(dq=A16 * 5 + 16), ta.ATTN_ERR_ALIAS),
    (dict(causal=3), ta.ATTN_ERR_MASK),
])
def test_bwd_noalloc_argument_errors_return_before_any_hip_call(lib, kw, status):
    assert call_bwd_noalloc(**kw) == status


def test_bwd_noalloc_limit_is_exactly_2_pow_20_rows(lib):
    # exactly 2^20 rows passes the size check (and then fails on a later
    # argument check, still before any HIP call); one more row does not
    assert call_bwd_noalloc(B=1, H=16, N_q=65536, dout=0) == ta.ATTN_ERR_NULL
    assert call_bwd_noalloc(B=1, H=16, N_q=65537, dout=0) == ta.ATTN_ERR_SCRATCH


def test_bwd_noalloc_empty_problem_is_a_noop(lib):
    assert call_bwd_noalloc(B=0, q=0, k=0, v=0, o=0, dout=0, lse=0, dq=0, dk=0, dv=0) == ta.ATTN_OK
    assert call_bwd_noalloc(N_q=0, N_k=0, q=0, k=0, v=0, o=0, dout=0, lse=0, dq=0, dk=0, dv=0) == ta.ATTN_OK
