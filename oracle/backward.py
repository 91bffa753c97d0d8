"""Plain fp64 CPU oracle for the attention backward pass (dQ, dK, dV).

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import this module:
only the tests and ``bench.py``'s ``cpu_baseline`` leg use it. It shares no
code with the HIP library.

Page cited: [PT2CUDA] aiknowledge.cn, "4.5 注意力优化实战：从PyTorch到CUDA的完整流程",
step 4.2 (backward kernel): the backward pass propagates the gradient of the
output to Q, K and V; dQ takes every K/V block, dK and dV take every Q block,
and the softmax of the forward pass is needed again (recomputed from what the
forward kept). The pages give no formulas, so this module writes out the
chain rule through the forward definition of ``oracle.attention``:

  S  = scale * Q K^T, masked entries -inf;   P = softmax_rows(S)  (0 on a
  fully masked row);   O = P V.
  For a scalar loss with upstream gradient dO = dL/dO:
    dV = P^T dO
    dP = dO V^T
    dS = P * (dP - rowsum(P * dP))       (the softmax Jacobian, row by row)
    dQ = scale * dS K
    dK = scale * dS^T Q
  Masked entries have P = 0 and so dS = 0: they pass no gradient, and a
  fully masked row gives a zero dQ row and adds nothing to dK or dV.

Parity status: pinned in ``tests/test_oracle_bwd.py`` by central finite
differences of the forward oracle, by invariants (the dK rows of a head sum to
zero, dO = 0 gives zero gradients, V with equal rows gives dQ = dK = 0), by a
closed form (Q = 0: dV_j is the sum of dO_i / n_i over the rows i that see key
j) and by torch's fp64 autograd on CPU as a library cross-check.
"""
from __future__ import annotations

from typing import Optional

import numpy as np

from .attention import attention


def attention_bwd(q: np.ndarray, k: np.ndarray, v: np.ndarray, dout: np.ndarray, scale: float,
                  causal: bool = False, seqlens_k: Optional[np.ndarray] = None,
                  q_start: Optional[np.ndarray] = None, attn_mask: Optional[np.ndarray] = None):
    """Gradients (dQ, dK, dV) of attention in float64, shapes of q, k, v.

    Rows and keys follow the masking rules of ``oracle.attention``
    (causal, keys j < seqlens_k[b], rows i >= q_start[b], the boolean attn_mask).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    g = np.asarray(dout, dtype=np.float64)
    B, H, n_q, d = q.shape
    n_k = k.shape[2]
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    if n_k == 0 or n_q == 0:
        return dq, dk, dv
    sc = np.float64(scale)
    # P of the forward definition, every row at once (the oracle's own forward)
    _, _, p = attention(q, k, v, scale, causal, seqlens_k=seqlens_k, q_start=q_start, return_probs=True,
                        attn_mask=attn_mask)
    for b in range(B):
        for h in range(H):
            pb = p[b, h]                                   # [n_q, n_k]
            dv[b, h] = pb.T @ g[b, h]
            dp = g[b, h] @ v[b, h].T                       # [n_q, n_k]
            ds = pb * (dp - (pb * dp).sum(axis=1, keepdims=True))
            dq[b, h] = sc * (ds @ k[b, h])
            dk[b, h] = sc * (ds.T @ q[b, h])
    return dq, dk, dv
