"""Plain fp64 CPU oracle for the FP8 attention forward - TEST INFRASTRUCTURE.

Only the tests, ``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline``
leg may import this module. It shares no code with the HIP library.

Page cited: [MEMWALL] codechina.net, "GPU 内存墙 ... FlashAttention" article,
section 9 (future directions), mixed-precision item: the two matrix products
of attention taken in FP8 with a wider accumulator. The page gives no
formulas; the readings taken here are:
  * the FP8 format is OCP E4M3 ("e4m3fn": 1 sign bit, 4 exponent bits with
    bias 7, 3 mantissa bits, subnormals, no infinities, S.1111.111 = NaN);
  * Q, K and V arrive already quantized, each with one fp32 descale factor
    per tensor: the real tensor is decode(codes) * descale;
  * V arrives transposed, [B, H, d, N_k] (key index fastest);
  * what the method computes is then attention (the definition in
    ``oracle.attention``) of the dequantized tensors, scores times ``scale``.
    Rounding the probabilities to FP8 before the second product is an
    approximation of that definition, covered by the tolerance of the test,
    not part of this oracle.

Parity status: ``e4m3_decode`` is pinned by the format's defining values
(1.0, 448, the smallest normal and subnormal, the NaN codes, the sign bit) and
by torch's float8_e4m3fn conversion as a separate library; ``attention_fp8``
by closed forms on its inputs (Q = 0 gives the mean of the visible V rows,
V with equal rows gives that row) and by the descale invariances
(tests/test_oracle_fp8.py).
"""
from __future__ import annotations

from typing import Optional

import numpy as np

from .attention import attention


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    """Decode OCP E4M3 bytes (uint8) to float64, exactly.

    value = (-1)^s * 2^(e - 7) * (1 + m / 8) for exponent field e > 0,
            (-1)^s * 2^(-6) * (m / 8)       for e = 0 (subnormal),
    and NaN for e = 15, m = 7 (no infinities in this format).
    """
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    s = (c >> 7) & 1
    e = (c >> 3) & 15
    m = c & 7
    mag = np.where(e > 0, np.ldexp(1.0 + m / 8.0, e - 7), np.ldexp(m / 8.0, -6))
    out = np.where(s == 1, -mag, mag)
    return np.where((e == 15) & (m == 7), np.nan, out)


def attention_fp8(q8: np.ndarray, k8: np.ndarray, vt8: np.ndarray, scale: float, q_descale: float,
                  k_descale: float, v_descale: float, causal=False,
                  seqlens_k: Optional[np.ndarray] = None, rows=None):
    """(O, LSE) in float64 of attention over the dequantized FP8 inputs.

    q8 [B, H, N_q, d], k8 [B, H, N_k, d], vt8 [B, H, d, N_k]: uint8 E4M3 codes.
    ``causal``, ``seqlens_k`` and ``rows`` follow ``oracle.attention``.
    """
    q = e4m3_decode(q8) * np.float64(q_descale)
    k = e4m3_decode(k8) * np.float64(k_descale)
    v = np.swapaxes(e4m3_decode(vt8), -1, -2) * np.float64(v_descale)
    return attention(q, k, v, scale, causal, seqlens_k=seqlens_k, rows=rows)
