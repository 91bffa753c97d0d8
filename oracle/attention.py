"""Plain fp64 CPU oracle for the attention forward pass.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import this module:
only the tests, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` use it. It shares no code with the HIP library.

Pages cited (their sections, not line numbers):
  [PT2CUDA]  aiknowledge.cn, "4.5 注意力优化实战：从PyTorch到CUDA的完整流程"
             (attention optimisation in practice, from PyTorch to CUDA).
  [MEMWALL]  codechina.net, "GPU 内存墙 ... FlashAttention" article.
  [PROFILE3] "Profiling in PyTorch (part 3): Attention is all you profile"
             (Chinese translation, feinterview.poetries.top).

Two implementations live here, both in float64:
  * ``attention`` - the unfused definition (scores, scale, mask, two-pass
    softmax, weighted sum). This is the oracle proper.
  * ``attention_online`` - the tiled online-softmax recurrence, written from
    the pages' description, used only to pin the definition (the pages state
    the two agree exactly in exact arithmetic).

Readings of the pages taken here (each also listed in the design notes):
  * masked scores are -inf and carry exactly zero weight; a row whose keys
    are all masked outputs O = 0 and LSE = -inf (the NaN-safe softmax the
    SDPA math backend uses, [PROFILE3] math-backend section);
  * the scale multiplies the scores before masking ([PT2CUDA] step 1 and
    [PROFILE3] naive module order), so scale = 0 never forms 0 * -inf;
  * causal means key j is visible to query i iff j <= i, the lower-triangular
    [seq, seq] mask of [PROFILE3] (top-left aligned when N_q != N_k); causal = 2
    aligns the triangle bottom-right instead (j <= i + N_k - N_q), the pages'
    mask when the queries are the last N_q positions of the key sequence;
  * variable-length keys are masked through a per-batch valid length
    ([MEMWALL] §6.2), clamped to [0, N_k]; a per-batch count of leading query
    rows that attend to nothing (``q_start``, clamped to [0, N_q]) lets a
    partial block of rows be fully masked;
  * LSE is the natural-log log-sum-exp of the scaled, masked scores (the pages
    do not define it; the backward pass of [PT2CUDA] step 4.2 needs the softmax
    denominator, which this carries).
"""
from __future__ import annotations

from typing import Optional, Sequence

import numpy as np


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Expand bfloat16 bit patterns (uint16) to float64 exactly."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


def causal_offset(n_q: int, n_k: int, causal) -> int:
    """Diagonal offset of a causal mask: key j is visible to row i iff j <= i + offset.

    causal = 1 (or True): top-left aligned, offset 0 (the lower triangle of
    [PROFILE3]); causal = 2: bottom-right aligned, offset n_k - n_q, so the
    last query row sees every key (rows are the last n_q positions of the
    key sequence, as when new queries attend to a cache of earlier keys).
    """
    return n_k - n_q if int(causal) == 2 else 0


def allowed_mask(n_q: int, n_k: int, causal, kv_len: Optional[int] = None,
                 q_start: Optional[int] = None, rows: Optional[Sequence[int]] = None) -> np.ndarray:
    """Boolean [R, n_k] matrix, True where query row i may attend to key j.

    Built explicitly, entry by entry, from the three rules:
      causal   -> j <= i + causal_offset(...), the lower triangle ([PROFILE3],
                  math-backend mask built with ones -> tril), top-left
                  (causal = 1) or bottom-right (causal = 2) aligned;
      kv_len   -> j < kv_len, keys past a sequence's valid length are masked
                  ([MEMWALL] §6.2, masks mark the valid positions);
      q_start  -> i >= q_start, leading rows see no key at all.
    """
    kv = n_k if kv_len is None else int(min(max(int(kv_len), 0), n_k))
    qs = 0 if q_start is None else int(min(max(int(q_start), 0), n_q))
    i = np.arange(n_q) if rows is None else np.asarray(rows, dtype=np.int64)
    j = np.arange(n_k)
    ok = (j[None, :] < kv) & (i[:, None] >= qs)
    if causal:
        ok &= j[None, :] <= i[:, None] + causal_offset(n_q, n_k, causal)
    return ok


def _rows_blocks(rows: np.ndarray, block: int):
    for s in range(0, rows.shape[0], block):
        yield rows[s:s + block]


def dense_allowed(attn_mask: Optional[np.ndarray], b: int, h: int, rows: np.ndarray) -> Optional[np.ndarray]:
    """Rows ``rows`` of the boolean mask for (b, h), or None without a mask.

    ``attn_mask`` is boolean, broadcastable to [B, H, N_q, N_k], True where
    row i may attend to key j (the SDPA convention for a boolean mask,
    [PROFILE3]; [PT2CUDA] step 1 writes the same rule as scores where the mask
    is 0 becoming -inf). It is intersected with the rule masks.
    """
    if attn_mask is None:
        return None
    m = np.asarray(attn_mask, dtype=bool)
    return m[b if m.shape[0] > 1 else 0, h if m.shape[1] > 1 else 0][rows]


def expand_block_mask(block_mask: np.ndarray, n_q: int, n_k: int, block_q: int, block_k: int) -> np.ndarray:
    """Boolean [.., n_q, n_k] mask from a block mask [.., ceil(n_q/block_q), ceil(n_k/block_k)]:
    entry (i, j) is the flag of block (i // block_q, j // block_k).

    Block-sparse attention ([MEMWALL] §7) computes only the blocks whose flag is
    set; in exact arithmetic that is attention under this expanded mask.
    """
    bm = np.asarray(block_mask, dtype=bool)
    return bm[..., np.arange(n_q) // block_q, :][..., np.arange(n_k) // block_k]


def attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float, causal: bool = False,
              seqlens_k: Optional[np.ndarray] = None, q_start: Optional[np.ndarray] = None,
              rows: Optional[Sequence[int]] = None, return_probs: bool = False, row_block: int = 1024,
              attn_mask: Optional[np.ndarray] = None):
    """Unfused scaled-dot-product attention in float64.

    q: [B, H, N_q, d]; k, v: [B, H, N_k, d] (float64, any values).
    Returns O [B, H, R, d_v] and LSE [B, H, R] for the R selected query rows
    (all rows when ``rows`` is None); with ``return_probs`` also P [B, H, R, N_k].

    Steps, per (b, h), following the unfused module of [PT2CUDA] step 1
    ("baseline implementation") and [PROFILE3] (naive attention):
      1. S = (Q K^T) * scale;
      2. S[not allowed] = -inf (``allowed_mask``);
      3. two-pass softmax ([MEMWALL] §3.1): m = max_j S, E = exp(S - m),
         l = sum_j E, P = E / l; a row with m = -inf has P = 0
         ([PROFILE3], the math backend's NaN-safe softmax);
      4. O = P V and LSE = m + ln l (-inf for a fully masked row).
    Rows are processed in blocks of ``row_block`` to bound memory; every
    row's softmax is still taken over all of its keys at once.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, H, n_q, d = q.shape
    n_k = k.shape[2]
    sel = np.arange(n_q) if rows is None else np.asarray(rows, dtype=np.int64)
    R = sel.shape[0]
    out = np.zeros((B, H, R, v.shape[3]), dtype=np.float64)
    lse = np.full((B, H, R), -np.inf, dtype=np.float64)
    probs = np.zeros((B, H, R, n_k), dtype=np.float64) if return_probs else None
    if n_k == 0:   # no keys at all: every row is fully masked
        return (out, lse, probs) if return_probs else (out, lse)
    sc = np.float64(scale)
    for b in range(B):
        kv = None if seqlens_k is None else int(seqlens_k[b])
        qs = None if q_start is None else int(q_start[b])
        for h in range(H):
            pos = 0
            for blk in _rows_blocks(sel, row_block):
                r = blk.shape[0]
                s = (q[b, h, blk] @ k[b, h].T) * sc
                ok = allowed_mask(n_q, n_k, causal, kv, qs, rows=blk)
                dm = dense_allowed(attn_mask, b, h, blk)
                if dm is not None:
                    ok = ok & dm
                s[~ok] = -np.inf
                m = s.max(axis=1)
                live = m > -np.inf
                e = np.zeros_like(s)
                with np.errstate(invalid="ignore", over="ignore"):
                    e[live] = np.exp(s[live] - m[live, None])
                l = e.sum(axis=1)
                p = np.zeros_like(s)
                p[live] = e[live] / l[live, None]
                # keys at or past the valid length carry no weight and their
                # contents (padding) are never used
                n_valid = n_k if kv is None else min(max(kv, 0), n_k)
                out[b, h, pos:pos + r] = p[:, :n_valid] @ v[b, h, :n_valid]
                lse[b, h, pos:pos + r][live] = m[live] + np.log(l[live])
                if probs is not None:
                    probs[b, h, pos:pos + r] = p
                pos += r
    if return_probs:
        return out, lse, probs
    return out, lse


def attention_online(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float, causal: bool = False,
                     seqlens_k: Optional[np.ndarray] = None, q_start: Optional[np.ndarray] = None,
                     block_k: int = 64):
    """The tiled online-softmax recurrence in float64, for pinning ``attention``.

    Follows [PT2CUDA] step 3.1 ("math basis: tiled attention") and [MEMWALL]
    §3.2 ("Online Softmax"): for each query row keep a running max m, a running
    sum l and an unnormalised output o; for each key block j, with the block's
    scaled, masked scores s:
        m_new = max(m, rowmax(s))
        alpha = exp(m - m_new)                 (correction of the old terms)
        p     = exp(s - m_new)
        l     = alpha * l + rowsum(p)
        o     = alpha * o + p @ V_j
        m     = m_new
    and at the end O = o / l. Reading taken where the pages are silent: while a
    row has seen only masked keys, m_new is -inf and exp(-inf - -inf) is
    undefined, so the subtraction uses 0 in place of an infinite m_new; masked
    scores then contribute exp(-inf) = 0 and alpha = exp(-inf) = 0, and a row
    that never sees a key ends with l = 0, O = 0, LSE = -inf.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, H, n_q, d = q.shape
    n_k = k.shape[2]
    sc = np.float64(scale)
    out = np.zeros((B, H, n_q, v.shape[3]))
    lse = np.full((B, H, n_q), -np.inf)
    if n_k == 0:
        return out, lse
    for b in range(B):
        kv = None if seqlens_k is None else int(seqlens_k[b])
        qs = None if q_start is None else int(q_start[b])
        ok_full = allowed_mask(n_q, n_k, causal, kv, qs)
        n_valid = n_k if kv is None else min(max(kv, 0), n_k)
        for h in range(H):
            m = np.full(n_q, -np.inf)
            l = np.zeros(n_q)
            o = np.zeros((n_q, v.shape[3]))
            for j0 in range(0, n_k, block_k):
                j1 = min(j0 + block_k, n_k)
                s = (q[b, h] @ k[b, h, j0:j1].T) * sc
                s[~ok_full[:, j0:j1]] = -np.inf
                m_new = np.maximum(m, s.max(axis=1))
                m_sub = np.where(np.isneginf(m_new), 0.0, m_new)
                alpha = np.exp(m - m_sub)
                p = np.exp(s - m_sub[:, None])
                l = alpha * l + p.sum(axis=1)
                # keys past the valid length: zero weight, contents never used
                vj = v[b, h, j0:j1].copy()
                vj[np.arange(j0, j1) >= n_valid] = 0.0
                o = alpha[:, None] * o + p @ vj
                m = m_new
            live = l > 0
            out[b, h][live] = o[live] / l[live, None]
            lse[b, h][live] = m[live] + np.log(l[live])
    return out, lse
