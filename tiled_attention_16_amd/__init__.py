"""Python binding of the MI355X fused attention library (``libattn.so``).

Argument marshalling only: every step of the computation runs in the HIP
kernels behind ``attn_fwd`` and ``attn_bwd`` in ``include/attn.h``. PyTorch supplies device
memory and the current stream. There is no fallback: if the library is
missing or the tensors are not on a GPU, the call raises.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional, Tuple

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libattn.so")

ATTN_OK = 0
ATTN_ERR_NULL = 1
ATTN_ERR_SHAPE = 2
ATTN_ERR_HEAD_DIM = 3
ATTN_ERR_SCALE = 4
ATTN_ERR_ALIGN = 5
ATTN_ERR_ALIAS = 6
ATTN_ERR_LAUNCH = 7
ATTN_ERR_MASK = 8
ATTN_ERR_SCRATCH = 9

# causal modes of the C ABI
CAUSAL_NONE, CAUSAL_TOP_LEFT, CAUSAL_BOTTOM_RIGHT = 0, 1, 2


def causal_mode(causal) -> int:
    """Map ``False``/``True``/``"top_left"``/``"bottom_right"`` (or 0/1/2) to the ABI's causal mode."""
    if isinstance(causal, str):
        modes = {"none": 0, "top_left": 1, "bottom_right": 2}
        if causal not in modes:
            raise ValueError(f"causal must be one of {sorted(modes)}, got {causal!r}")
        return modes[causal]
    return int(causal)

# every symbol include/attn.h declares
EXPORTS = ("attn_bwd", "attn_bwd_block_sparse", "attn_bwd_masked", "attn_bwd_noalloc", "attn_fwd", "attn_fwd_block_sparse",
           "attn_fwd_fp8", "attn_fwd_masked", "attn_mask_pack", "attn_status_str", "attn_version")

SPARSE_BLOCK_Q = 256   # query rows per block of attn_fwd_block_sparse's block mask
SPARSE_BLOCK_K = 128   # keys per block

_lib = None


def load_library() -> ctypes.CDLL:
    """Load ``libattn.so`` (built by ``tiled_attention_16_amd.build``); raise if absent."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(f"{_LIB_PATH} is missing: build it with `python -m tiled_attention_16_amd.build`")
    lib = ctypes.CDLL(_LIB_PATH)
    lib.attn_fwd.restype = ctypes.c_int
    lib.attn_fwd.argtypes = [
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
        ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
        ctypes.c_float, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
    ]
    lib.attn_fwd_masked.restype = ctypes.c_int
    lib.attn_fwd_masked.argtypes = lib.attn_fwd.argtypes[:14] + [ctypes.c_void_p, ctypes.c_longlong, ctypes.c_longlong,
                                                                 ctypes.c_int, ctypes.c_void_p]
    lib.attn_fwd_block_sparse.restype = ctypes.c_int
    lib.attn_fwd_block_sparse.argtypes = lib.attn_fwd.argtypes[:14] + [ctypes.c_void_p, ctypes.c_longlong,
                                                                       ctypes.c_longlong, ctypes.c_void_p]
    lib.attn_mask_pack.restype = ctypes.c_int
    lib.attn_mask_pack.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_longlong, ctypes.c_int, ctypes.c_int,
                                   ctypes.c_void_p]
    lib.attn_bwd.restype = ctypes.c_int
    lib.attn_bwd.argtypes = [ctypes.c_void_p] * 10 + [ctypes.c_int] * 5 + [ctypes.c_float, ctypes.c_int] + \
        [ctypes.c_void_p] * 3
    lib.attn_bwd_noalloc.restype = ctypes.c_int
    lib.attn_bwd_noalloc.argtypes = [ctypes.c_void_p] * 9 + [ctypes.c_int] * 5 + [ctypes.c_float, ctypes.c_int] + \
        [ctypes.c_void_p] * 3
    lib.attn_bwd_masked.restype = ctypes.c_int
    lib.attn_bwd_masked.argtypes = lib.attn_bwd.argtypes[:19] + [ctypes.c_void_p, ctypes.c_longlong,
                                                                 ctypes.c_longlong, ctypes.c_int, ctypes.c_void_p]
    lib.attn_bwd_block_sparse.restype = ctypes.c_int
    lib.attn_bwd_block_sparse.argtypes = lib.attn_bwd.argtypes[:19] + [ctypes.c_void_p, ctypes.c_longlong,
                                                                       ctypes.c_longlong, ctypes.c_void_p]
    lib.attn_fwd_fp8.restype = ctypes.c_int
    lib.attn_fwd_fp8.argtypes = [ctypes.c_void_p] * 3 + [ctypes.c_longlong] + [ctypes.c_void_p] * 2 + \
        [ctypes.c_int] * 5 + [ctypes.c_float] * 4 + [ctypes.c_int, ctypes.c_void_p]
    lib.attn_status_str.restype = ctypes.c_char_p
    lib.attn_status_str.argtypes = [ctypes.c_int]
    lib.attn_version.restype = ctypes.c_int
    lib.attn_version.argtypes = []
    _lib = lib
    return lib


def attn_status_str(status: int) -> str:
    return load_library().attn_status_str(int(status)).decode()


def attn_version() -> int:
    return int(load_library().attn_version())


class AttnError(RuntimeError):
    def __init__(self, status: int, name: str = "attn_fwd"):
        super().__init__(f"{name} failed: {attn_status_str(status)} (status {status})")
        self.status = status


def attn_fwd_raw(q: int, k: int, v: int, o: int, lse: int, B: int, H: int, N_q: int, N_k: int, d: int,
                 scale: float, causal: bool, seqlens_k: int, q_start: int, stream: int) -> int:
    """The C entry point with plain integers for pointers; returns the status code."""
    return int(load_library().attn_fwd(q or None, k or None, v or None, o or None, lse or None,
                                       int(B), int(H), int(N_q), int(N_k), int(d), ctypes.c_float(scale),
                                       causal_mode(causal), seqlens_k or None, q_start or None, stream or None))


def mask_row_words(N_k: int) -> int:
    """Words per row of a packed mask: ceil(N_k / 32) rounded up to a multiple of 8."""
    return max(8, ((N_k + 255) // 256) * 8)


def pack_mask(mask, stream=None):
    """Pack a boolean (or uint8) GPU mask ``[Bm, Hm, N_q, N_k]`` (True = may attend)
    into the bit layout of ``attn_fwd_masked`` with ``attn_mask_pack``.

    Returns ``(bits, mask_stride_b, mask_stride_h, row_words)``; a size-1
    batch or head dimension becomes a zero stride (broadcast).
    """
    import torch

    lib = load_library()
    if not isinstance(mask, torch.Tensor) or not mask.is_cuda or mask.dim() != 4 or \
            mask.dtype not in (torch.bool, torch.uint8):
        raise ValueError("mask must be a bool or uint8 GPU tensor [B or 1, H or 1, N_q, N_k]")
    m = mask.contiguous()
    if m.dtype == torch.bool:
        m = m.view(torch.uint8)
    Bm, Hm, N_q, N_k = m.shape
    rw = mask_row_words(N_k)
    bits = torch.empty((Bm, Hm, N_q, rw), dtype=torch.int32, device=m.device)
    st = stream if stream is not None else torch.cuda.current_stream(m.device)
    status = lib.attn_mask_pack(m.data_ptr() or None, bits.data_ptr() or None, Bm * Hm * N_q, N_k, rw,
                                ctypes.c_void_p(st.cuda_stream))
    if status != ATTN_OK:
        raise AttnError(status, "attn_mask_pack")
    return bits, (0 if Bm == 1 else Hm * N_q * rw), (0 if Hm == 1 else N_q * rw), rw


def _block_mask_args(block_mask, B, H, N_q, N_k):
    """Check a block mask and return (uint8 tensor, batch stride, head stride) in bytes."""
    import torch

    nqb, nkb = -(-N_q // SPARSE_BLOCK_Q), -(-N_k // SPARSE_BLOCK_K)
    if not isinstance(block_mask, torch.Tensor) or not block_mask.is_cuda or block_mask.dim() != 4 or \
            block_mask.dtype not in (torch.bool, torch.uint8) or block_mask.shape[2:] != (nqb, nkb) or \
            block_mask.shape[0] not in (1, B) or block_mask.shape[1] not in (1, H):
        raise ValueError(f"block_mask must be a bool/uint8 GPU tensor [1 or {B}, 1 or {H}, {nqb}, {nkb}]")
    bm = block_mask.contiguous()
    if bm.dtype == torch.bool:
        bm = bm.view(torch.uint8)
    sb = 0 if bm.shape[0] == 1 else bm.shape[1] * nqb * nkb
    sh = 0 if bm.shape[1] == 1 else nqb * nkb
    return bm, sb, sh


def attn_fwd(q, k, v, *, causal: bool = False, scale: Optional[float] = None, seqlens_k=None, q_start=None,
             return_lse: bool = True, out=None, lse=None, stream=None, attn_mask=None,
             packed_mask=None, block_mask=None) -> Tuple[object, Optional[object]]:
    """Fused attention forward on bf16 ``[B, H, N, d]`` CUDA (HIP) tensors.

    ``causal``: False (none), True or "top_left" (key j visible to row i iff
    j <= i), "bottom_right" (iff j <= i + N_k - N_q). ``attn_mask``: optional
    bool GPU tensor ``[B or 1, H or 1, N_q, N_k]``, True = may attend,
    intersected with the other rules (packed by the library on each call;
    pass ``packed_mask=pack_mask(m)`` to pack once). ``block_mask``: optional
    bool/uint8 GPU tensor ``[B or 1, H or 1, ceil(N_q/256), ceil(N_k/128)]``;
    only the blocks it keeps are computed (``attn_fwd_block_sparse``).
    Returns ``(o, lse)``; ``lse`` is None unless ``return_lse``. ``scale``
    defaults to ``d ** -0.5``. ``seqlens_k`` / ``q_start`` are optional int32
    device tensors of shape ``[B]``. The kernel is launched on ``stream`` (a
    ``torch.cuda.Stream``) or on torch's current stream.
    """
    import torch

    lib = load_library()
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not isinstance(t, torch.Tensor) or t.dtype != torch.bfloat16 or not t.is_cuda:
            raise ValueError(f"{name} must be a bfloat16 GPU tensor")
        if t.dim() != 4 or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous [B, H, N, d] tensor")
    B, H, N_q, d = q.shape
    if k.shape[:2] != (B, H) or k.shape[3] != d or v.shape != k.shape:
        raise ValueError(f"shape mismatch: q {tuple(q.shape)} k {tuple(k.shape)} v {tuple(v.shape)}")
    N_k = k.shape[2]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    for name, t in (("seqlens_k", seqlens_k), ("q_start", q_start)):
        if t is not None and (t.dtype != torch.int32 or not t.is_cuda or t.numel() != B or not t.is_contiguous()):
            raise ValueError(f"{name} must be a contiguous int32 GPU tensor of {B} elements")
    if out is None:
        out = torch.empty_like(q)
    elif out.shape != q.shape or out.dtype != torch.bfloat16 or not out.is_contiguous():
        raise ValueError("out must be a contiguous bf16 tensor shaped like q")
    if return_lse and lse is None:
        lse = torch.empty((B, H, N_q), dtype=torch.float32, device=q.device)
    if lse is not None and (lse.shape != (B, H, N_q) or lse.dtype != torch.float32 or not lse.is_contiguous()):
        raise ValueError("lse must be a contiguous float32 [B, H, N_q] tensor")
    st = stream if stream is not None else torch.cuda.current_stream(q.device)
    if attn_mask is not None and packed_mask is None:
        if attn_mask.dim() != 4 or attn_mask.shape[2:] != (N_q, N_k) or attn_mask.shape[0] not in (1, B) or \
                attn_mask.shape[1] not in (1, H):
            raise ValueError(f"attn_mask must be [1 or {B}, 1 or {H}, {N_q}, {N_k}]")
        packed_mask = pack_mask(attn_mask, stream=st)
    args = [q.data_ptr() or None, k.data_ptr() or None, v.data_ptr() or None, out.data_ptr() or None,
            (lse.data_ptr() or None) if lse is not None else None, B, H, N_q, N_k, d, ctypes.c_float(scale),
            causal_mode(causal), seqlens_k.data_ptr() if seqlens_k is not None else None,
            q_start.data_ptr() if q_start is not None else None]
    if block_mask is not None:
        if packed_mask is not None:
            raise ValueError("block_mask and attn_mask cannot be combined")
        bm, sb, sh = _block_mask_args(block_mask, B, H, N_q, N_k)
        status = lib.attn_fwd_block_sparse(*args, bm.data_ptr(), sb, sh, ctypes.c_void_p(st.cuda_stream))
    elif packed_mask is not None:
        bits, sb, sh, rw = packed_mask
        status = lib.attn_fwd_masked(*args, bits.data_ptr() or None, sb, sh, rw, ctypes.c_void_p(st.cuda_stream))
    else:
        status = lib.attn_fwd(*args, ctypes.c_void_p(st.cuda_stream))
    if status != ATTN_OK:
        raise AttnError(status)
    return out, (lse if return_lse else None)


def attn_bwd_raw(q: int, k: int, v: int, o: int, dout: int, lse: int, dq: int, dk: int, dv: int, delta: int,
                 B: int, H: int, N_q: int, N_k: int, d: int, scale: float, causal: bool, seqlens_k: int,
                 q_start: int, stream: int) -> int:
    """The C entry point ``attn_bwd`` with plain integers for pointers; returns the status code."""
    p = [x or None for x in (q, k, v, o, dout, lse, dq, dk, dv, delta)]
    return int(load_library().attn_bwd(*p, int(B), int(H), int(N_q), int(N_k), int(d), ctypes.c_float(scale),
                                       causal_mode(causal), seqlens_k or None, q_start or None, stream or None))


def attn_bwd(q, k, v, o, lse, dout, *, causal: bool = False, scale: Optional[float] = None, seqlens_k=None,
             q_start=None, dq=None, dk=None, dv=None, delta=None, stream=None, attn_mask=None, packed_mask=None,
             block_mask=None):
    """Gradients ``(dq, dk, dv)`` of ``attn_fwd`` for upstream gradient ``dout``.

    ``o`` and ``lse`` are ``attn_fwd``'s outputs for the same inputs, mask and
    scale. All tensors are contiguous GPU tensors: q, o, dout bf16
    ``[B, H, N_q, d]``; k, v bf16 ``[B, H, N_k, d]``; lse float32 ``[B, H, N_q]``.
    ``delta`` (float32 ``[B, H, N_q, 2]``) is the kernels' workspace; it is
    allocated here when not given. ``attn_mask`` / ``packed_mask``: the mask
    the forward used (see ``attn_fwd``).
    """
    import torch

    lib = load_library()
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o), ("dout", dout)):
        if not isinstance(t, torch.Tensor) or t.dtype != torch.bfloat16 or not t.is_cuda:
            raise ValueError(f"{name} must be a bfloat16 GPU tensor")
        if t.dim() != 4 or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous [B, H, N, d] tensor")
    B, H, N_q, d = q.shape
    if k.shape[:2] != (B, H) or k.shape[3] != d or v.shape != k.shape:
        raise ValueError(f"shape mismatch: q {tuple(q.shape)} k {tuple(k.shape)} v {tuple(v.shape)}")
    if o.shape != q.shape or dout.shape != q.shape:
        raise ValueError("o and dout must be shaped like q")
    N_k = k.shape[2]
    if not isinstance(lse, torch.Tensor) or lse.dtype != torch.float32 or not lse.is_cuda or \
            lse.shape != (B, H, N_q) or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous float32 [B, H, N_q] GPU tensor")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    for name, t in (("seqlens_k", seqlens_k), ("q_start", q_start)):
        if t is not None and (t.dtype != torch.int32 or not t.is_cuda or t.numel() != B or not t.is_contiguous()):
            raise ValueError(f"{name} must be a contiguous int32 GPU tensor of {B} elements")
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    for name, t, ref in (("dq", dq, q), ("dk", dk, k), ("dv", dv, v)):
        if t.shape != ref.shape or t.dtype != torch.bfloat16 or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous bf16 tensor shaped like {name[1:]}")
    if delta is None:
        delta = torch.empty((B, H, N_q, 2), dtype=torch.float32, device=q.device)
    elif delta.shape != (B, H, N_q, 2) or delta.dtype != torch.float32 or not delta.is_contiguous():
        raise ValueError("delta must be a contiguous float32 [B, H, N_q, 2] tensor")
    st = stream if stream is not None else torch.cuda.current_stream(q.device)
    ptr = lambda t: t.data_ptr() or None  # noqa: E731
    if attn_mask is not None and packed_mask is None:
        packed_mask = pack_mask(attn_mask, stream=st)
    args = [ptr(q), ptr(k), ptr(v), ptr(o), ptr(dout), ptr(lse), ptr(dq), ptr(dk), ptr(dv), ptr(delta), B, H, N_q,
            N_k, d, ctypes.c_float(scale), causal_mode(causal), seqlens_k.data_ptr() if seqlens_k is not None else None,
            q_start.data_ptr() if q_start is not None else None]
    if block_mask is not None:
        if packed_mask is not None:
            raise ValueError("block_mask and attn_mask cannot be combined")
        bm, sb, sh = _block_mask_args(block_mask, B, H, N_q, N_k)
        status = lib.attn_bwd_block_sparse(*args, bm.data_ptr(), sb, sh, ctypes.c_void_p(st.cuda_stream))
    elif packed_mask is not None:
        bits, sb, sh, rw = packed_mask
        status = lib.attn_bwd_masked(*args, bits.data_ptr() or None, sb, sh, rw, ctypes.c_void_p(st.cuda_stream))
    else:
        status = lib.attn_bwd(*args, ctypes.c_void_p(st.cuda_stream))
    if status != ATTN_OK:
        raise AttnError(status, "attn_bwd")
    return dq, dk, dv


def attn_bwd_noalloc_raw(q: int, k: int, v: int, o: int, dout: int, lse: int, dq: int, dk: int, dv: int, B: int,
                         H: int, N_q: int, N_k: int, d: int, scale: float, causal, seqlens_k: int, q_start: int,
                         stream: int) -> int:
    """The C entry point ``attn_bwd_noalloc`` with plain integers for pointers; returns the status code."""
    p = [x or None for x in (q, k, v, o, dout, lse, dq, dk, dv)]
    return int(load_library().attn_bwd_noalloc(*p, int(B), int(H), int(N_q), int(N_k), int(d), ctypes.c_float(scale),
                                               causal_mode(causal), seqlens_k or None, q_start or None,
                                               stream or None))


def attn_bwd_noalloc(q, k, v, o, lse, dout, dq, dk, dv, *, causal: bool = False, scale: Optional[float] = None,
                     seqlens_k=None, q_start=None, stream=None):
    """``attn_bwd`` through the allocation-free entry point: the caller passes
    every output (``dq``, ``dk``, ``dv``), there is no ``delta`` workspace (the
    library keeps the row statistics in its own per-GPU array) and nothing is
    allocated. B*H*N_q is limited to 2**20 rows; calls that overlap in time on
    one GPU race. Returns ``(dq, dk, dv)``."""
    import torch

    lib = load_library()
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o), ("dout", dout), ("dq", dq), ("dk", dk), ("dv", dv)):
        if not isinstance(t, torch.Tensor) or t.dtype != torch.bfloat16 or not t.is_cuda:
            raise ValueError(f"{name} must be a bfloat16 GPU tensor")
        if t.dim() != 4 or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous [B, H, N, d] tensor")
    B, H, N_q, d = q.shape
    N_k = k.shape[2]
    if k.shape[:2] != (B, H) or k.shape[3] != d or v.shape != k.shape or dk.shape != k.shape or \
            dv.shape != k.shape or o.shape != q.shape or dout.shape != q.shape or dq.shape != q.shape:
        raise ValueError("shape mismatch among q, k, v, o, dout, dq, dk, dv")
    if not isinstance(lse, torch.Tensor) or lse.dtype != torch.float32 or not lse.is_cuda or \
            lse.shape != (B, H, N_q) or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous float32 [B, H, N_q] GPU tensor")
    for name, t in (("seqlens_k", seqlens_k), ("q_start", q_start)):
        if t is not None and (t.dtype != torch.int32 or not t.is_cuda or t.numel() != B or not t.is_contiguous()):
            raise ValueError(f"{name} must be a contiguous int32 GPU tensor of {B} elements")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    st = stream if stream is not None else torch.cuda.current_stream(q.device)
    ptr = lambda t: t.data_ptr() or None  # noqa: E731
    status = lib.attn_bwd_noalloc(ptr(q), ptr(k), ptr(v), ptr(o), ptr(dout), ptr(lse), ptr(dq), ptr(dk), ptr(dv),
                                  B, H, N_q, N_k, d, ctypes.c_float(scale), causal_mode(causal),
                                  seqlens_k.data_ptr() if seqlens_k is not None else None,
                                  q_start.data_ptr() if q_start is not None else None,
                                  ctypes.c_void_p(st.cuda_stream))
    if status != ATTN_OK:
        raise AttnError(status, "attn_bwd_noalloc")
    return dq, dk, dv


def attn_fwd_masked_raw(q: int, k: int, v: int, o: int, lse: int, B: int, H: int, N_q: int, N_k: int, d: int,
                        scale: float, causal, seqlens_k: int, q_start: int, mask_bits: int, mask_stride_b: int,
                        mask_stride_h: int, mask_row_words: int, stream: int) -> int:
    """The C entry point ``attn_fwd_masked`` with plain integers for pointers; returns the status code."""
    return int(load_library().attn_fwd_masked(q or None, k or None, v or None, o or None, lse or None, int(B), int(H),
                                              int(N_q), int(N_k), int(d), ctypes.c_float(scale), causal_mode(causal),
                                              seqlens_k or None, q_start or None, mask_bits or None,
                                              int(mask_stride_b), int(mask_stride_h), int(mask_row_words),
                                              stream or None))


def fp8_vt_stride(N_k: int) -> int:
    """Smallest row stride (bytes) of the transposed V that ``attn_fwd_fp8`` accepts."""
    return max(16, -(-N_k // 16) * 16)


def attn_fwd_fp8_raw(q: int, k: int, vt: int, vt_row_stride: int, o: int, lse: int, B: int, H: int, N_q: int,
                     N_k: int, d: int, scale: float, q_descale: float, k_descale: float, v_descale: float,
                     causal, stream: int) -> int:
    """The C entry point with plain integers for pointers; returns the status code."""
    return int(load_library().attn_fwd_fp8(q or None, k or None, vt or None, int(vt_row_stride), o or None,
                                           lse or None, int(B), int(H), int(N_q), int(N_k), int(d),
                                           ctypes.c_float(scale), ctypes.c_float(q_descale),
                                           ctypes.c_float(k_descale), ctypes.c_float(v_descale),
                                           causal_mode(causal), stream or None))


def attn_fwd_fp8(q8, k8, vt8, *, q_descale: float, k_descale: float, v_descale: float, causal=False,
                 scale: Optional[float] = None, return_lse: bool = True, out=None, lse=None,
                 stream=None) -> Tuple[object, Optional[object]]:
    """FP8 (OCP E4M3) attention forward on GPU tensors of E4M3 codes.

    ``q8`` ``[B, H, N_q, d]`` and ``k8`` ``[B, H, N_k, d]`` are uint8 or
    float8_e4m3fn tensors; ``vt8`` is V transposed, ``[B, H, d, S]`` with the
    row stride S a multiple of 16 and at least ``fp8_vt_stride(N_k)`` (bytes
    past N_k are ignored). The real tensors are codes times their descale.
    Returns ``(o, lse)``: bf16 ``[B, H, N_q, d]`` and fp32 ``[B, H, N_q]`` (None
    unless ``return_lse``). ``causal`` as in ``attn_fwd``; ``scale`` defaults
    to ``d ** -0.5``.
    """
    import torch

    lib = load_library()
    codes = []
    for name, t in (("q8", q8), ("k8", k8), ("vt8", vt8)):
        if not isinstance(t, torch.Tensor) or not t.is_cuda or t.dtype not in (torch.uint8, torch.float8_e4m3fn):
            raise ValueError(f"{name} must be a uint8 or float8_e4m3fn GPU tensor")
        if t.dim() != 4 or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous 4-d tensor")
        codes.append(t)
    B, H, N_q, d = q8.shape
    N_k = k8.shape[2]
    if k8.shape[:2] != (B, H) or k8.shape[3] != d or vt8.shape[:3] != (B, H, d):
        raise ValueError(f"shape mismatch: q8 {tuple(q8.shape)} k8 {tuple(k8.shape)} vt8 {tuple(vt8.shape)}")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty((B, H, N_q, d), dtype=torch.bfloat16, device=q8.device)
    elif out.shape != (B, H, N_q, d) or out.dtype != torch.bfloat16 or not out.is_contiguous():
        raise ValueError("out must be a contiguous bf16 tensor [B, H, N_q, d]")
    if return_lse and lse is None:
        lse = torch.empty((B, H, N_q), dtype=torch.float32, device=q8.device)
    if lse is not None and (lse.shape != (B, H, N_q) or lse.dtype != torch.float32 or not lse.is_contiguous()):
        raise ValueError("lse must be a contiguous float32 tensor [B, H, N_q]")
    st = stream if stream is not None else torch.cuda.current_stream(q8.device)
    status = lib.attn_fwd_fp8(q8.data_ptr() or None, k8.data_ptr() or None, vt8.data_ptr() or None, vt8.shape[3],
                              out.data_ptr() or None, lse.data_ptr() if lse is not None else None, B, H, N_q, N_k, d,
                              ctypes.c_float(scale), ctypes.c_float(q_descale), ctypes.c_float(k_descale),
                              ctypes.c_float(v_descale), causal_mode(causal), ctypes.c_void_p(st.cuda_stream))
    if status != ATTN_OK:
        raise AttnError(status, "attn_fwd_fp8")
    return out, (lse if return_lse else None)
