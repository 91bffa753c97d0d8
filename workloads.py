"""Seeded synthetic inputs for the attention forward pass.

This module is shared by the CPU oracle's tests and by the GPU path's tests and
benchmark. It only draws random numbers and encodes them as bfloat16 bit
patterns; it holds none of the attention arithmetic.

The pages describe random-tensor workloads in the ``[batch, heads, seq,
head_dim]`` layout at sequence lengths 2048/4096 and head dims 64/128
(codechina.net "GPU memory wall ... FlashAttention", §2.2 and the §5.2 table;
"Profiling in PyTorch (part 3)", flash-backend section). They name no dataset,
so every tensor here is iid Gaussian noise drawn from a fixed seed.

Recipe (the same for every shape):
  * one ``numpy.random.Generator(PCG64(seed))`` per workload;
  * draw Q, then K, then V as float32 standard normals in ``[B, H, N, d]``
    order, multiply by that tensor's standard deviation, round to bfloat16
    (round-to-nearest-even), keep the 16-bit patterns;
  * for a variable-length workload, draw ``seqlens_k`` after V with
    ``integers(lo, hi + 1, size=B)``; the rows masked through ``q_start`` are
    fixed by the workload, not drawn.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional, Sequence

import numpy as np


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); return uint16 bits.

    NaN inputs are not expected here (Gaussian draws are finite).
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> 16) & 1) + np.uint32(0x7FFF)
    return ((u + bias) >> 16).astype(np.uint16)


@dataclass(frozen=True)
class Workload:
    """One attention forward problem: shapes, mask rule and input distribution."""

    name: str
    B: int
    H: int
    N_q: int
    N_k: int
    d: int
    causal: bool
    seed: int
    sigma_q: float = 1.0
    sigma_k: float = 1.0
    sigma_v: float = 1.0
    # variable-length keys: seqlens_k[b] ~ U{lo..hi}; None = every key valid
    seqlens_range: Optional[tuple] = None
    # batches whose first ``q_start_rows`` query rows attend to nothing
    q_start_batches: Sequence[int] = field(default_factory=tuple)
    q_start_rows: int = 0

    @property
    def scale(self) -> np.float32:
        """Default softmax scale head_dim ** -0.5, as the float32 the kernel receives."""
        return np.float32(1.0 / np.sqrt(np.float64(self.d)))

    def flops(self) -> float:
        """Counted flops: 4*B*H*N_q*N_k*d, halved when causal (mask-independent otherwise)."""
        f = 4.0 * self.B * self.H * self.N_q * self.N_k * self.d
        return f / 2 if self.causal else f

    def algorithmic_bytes(self) -> float:
        """Q, K, V read once (bf16), O written once (bf16), LSE written once (fp32)."""
        return 2.0 * self.B * self.H * (self.N_q * self.d * 2 + self.N_k * self.d * 2) + 4.0 * self.B * self.H * self.N_q


# The five workloads of the benchmark statement, in order.
WORKLOADS = {
    "tiny_causal_d64": Workload("tiny_causal_d64", B=1, H=2, N_q=256, N_k=256, d=64, causal=True, seed=1001),
    "causal_n2048_d128": Workload("causal_n2048_d128", B=4, H=16, N_q=2048, N_k=2048, d=128, causal=True, seed=1002),
    "causal_n4096_d128": Workload("causal_n4096_d128", B=1, H=32, N_q=4096, N_k=4096, d=128, causal=True, seed=1003),
    "noncausal_n4096_d128": Workload("noncausal_n4096_d128", B=1, H=32, N_q=4096, N_k=4096, d=128, causal=False, seed=1003),
    "varlen_n1024_d64": Workload("varlen_n1024_d64", B=8, H=32, N_q=1024, N_k=1024, d=64, causal=False, seed=1004,
                                 seqlens_range=(256, 1024), q_start_batches=(1, 5), q_start_rows=64),
    "causal_n16384_d128_stress": Workload("causal_n16384_d128_stress", B=1, H=8, N_q=16384, N_k=16384, d=128,
                                          causal=True, seed=1005, sigma_q=2.0),
}

# Short sequences, where the kernel is bound by HBM bandwidth rather than by the
# matrix cores: for square shapes the counted flops per algorithmic byte are
# N/4 (causal) and N/2 (non-causal), 64 and 256 here, both below the MI355X
# ridge of about 312 flop/B (2.5 PFLOP/s over 8 TB/s). Each input set is over
# 500 MB, more than the 256 MB last-level cache.
HBM_PROBES = {
    "hbm_causal_n256_d128": Workload("hbm_causal_n256_d128", B=64, H=32, N_q=256, N_k=256, d=128, causal=True,
                                     seed=1006),
    "hbm_noncausal_n512_d128": Workload("hbm_noncausal_n512_d128", B=64, H=32, N_q=512, N_k=512, d=128,
                                        causal=False, seed=1007),
}

# The varlen workload's shape with every key valid and no masked rows: the
# reference its effective throughput is compared against (benchmark only).
REFERENCE = {
    "dense_n1024_d64": Workload("dense_n1024_d64", B=8, H=32, N_q=1024, N_k=1024, d=64, causal=False, seed=1004),
}

HEADLINE = "causal_n4096_d128"


@dataclass
class Inputs:
    """bf16 bit patterns (uint16) in [B, H, N, d] plus the optional int32 mask vectors."""

    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    seqlens_k: Optional[np.ndarray]
    q_start: Optional[np.ndarray]
    scale: np.float32
    causal: bool


def make_inputs(w: Workload) -> Inputs:
    """Draw the workload's tensors from its seed."""
    g = np.random.Generator(np.random.PCG64(w.seed))
    shp_q = (w.B, w.H, w.N_q, w.d)
    shp_k = (w.B, w.H, w.N_k, w.d)
    q = f32_to_bf16_bits(g.standard_normal(shp_q, dtype=np.float32) * np.float32(w.sigma_q))
    k = f32_to_bf16_bits(g.standard_normal(shp_k, dtype=np.float32) * np.float32(w.sigma_k))
    v = f32_to_bf16_bits(g.standard_normal(shp_k, dtype=np.float32) * np.float32(w.sigma_v))
    seqlens = None
    if w.seqlens_range is not None:
        lo, hi = w.seqlens_range
        seqlens = g.integers(lo, hi + 1, size=w.B).astype(np.int32)
    q_start = None
    if w.q_start_batches:
        q_start = np.zeros(w.B, dtype=np.int32)
        for b in w.q_start_batches:
            q_start[b] = w.q_start_rows
    return Inputs(q=q, k=k, v=v, seqlens_k=seqlens, q_start=q_start, scale=w.scale, causal=w.causal)


def make_random(B: int, H: int, N_q: int, N_k: int, d: int, seed: int, sigma=(1.0, 1.0, 1.0)):
    """Seeded bf16 Q, K, V bits for an arbitrary shape (edge-case tests)."""
    g = np.random.Generator(np.random.PCG64(seed))
    q = f32_to_bf16_bits(g.standard_normal((B, H, N_q, d), dtype=np.float32) * np.float32(sigma[0]))
    k = f32_to_bf16_bits(g.standard_normal((B, H, N_k, d), dtype=np.float32) * np.float32(sigma[1]))
    v = f32_to_bf16_bits(g.standard_normal((B, H, N_k, d), dtype=np.float32) * np.float32(sigma[2]))
    return q, k, v


def make_rising(B: int, H: int, N_q: int, N_k: int, d: int, seed: int, step: float = 0.5):
    """Seeded bf16 Q, K, V bits whose scores drift along the key axis.

    K row j is j*step times one fixed unit direction u plus N(0, 1) noise, so the
    score of query row i against key j grows (or shrinks) linearly in j with slope
    step * (q_i . u): rows with q_i . u > 0 see a new maximum in nearly every
    block of keys, the others keep the maximum of their first keys.
    """
    g = np.random.Generator(np.random.PCG64(seed))
    q = g.standard_normal((B, H, N_q, d), dtype=np.float32)
    u = g.standard_normal(d).astype(np.float32)
    u /= np.float32(np.linalg.norm(u))
    ramp = (np.arange(N_k, dtype=np.float32) * np.float32(step))[:, None] * u[None, :]
    k = g.standard_normal((B, H, N_k, d), dtype=np.float32) + ramp[None, None]
    v = g.standard_normal((B, H, N_k, d), dtype=np.float32)
    return f32_to_bf16_bits(q), f32_to_bf16_bits(k), f32_to_bf16_bits(v)



def make_dout(shape, seed: int, sigma: float = 1.0):
    """Seeded bf16 bits of an upstream gradient dO of the given shape (the
    backward pass's extra input): iid N(0, sigma^2), drawn after nothing else."""
    g = np.random.Generator(np.random.PCG64(seed))
    return f32_to_bf16_bits(g.standard_normal(tuple(shape), dtype=np.float32) * np.float32(sigma))


@dataclass
class Fp8Inputs:
    q8: np.ndarray          # uint8 E4M3 codes [B, H, N_q, d]
    k8: np.ndarray          # [B, H, N_k, d]
    vt8: np.ndarray         # V transposed: [B, H, d, N_k]
    q_descale: float
    k_descale: float
    v_descale: float


def make_fp8(B: int, H: int, N_q: int, N_k: int, d: int, seed: int, sigma=(1.0, 1.0, 1.0)) -> Fp8Inputs:
    """Seeded OCP E4M3 Q, K, V codes with one descale per tensor.

    Same draws as ``make_random`` (float32 normals times sigma, Q then K then
    V); each tensor is divided by amax / 448 (448 = the largest E4M3 value) and
    rounded to E4M3 by torch's float8_e4m3fn conversion; its descale is
    amax / 448. V is returned transposed, key index fastest.
    """
    import torch

    g = np.random.Generator(np.random.PCG64(seed))
    out = []
    for shape, s in (((B, H, N_q, d), sigma[0]), ((B, H, N_k, d), sigma[1]), ((B, H, N_k, d), sigma[2])):
        x = g.standard_normal(shape, dtype=np.float32) * np.float32(s)
        amax = float(np.abs(x).max()) if x.size else 1.0
        ds = amax / 448.0 if amax > 0 else 1.0
        y = np.clip(x.astype(np.float64) / ds, -448.0, 448.0).astype(np.float32)
        codes = torch.from_numpy(np.ascontiguousarray(y)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        out.append((codes, ds))
    (q8, qd), (k8, kd), (v8, vd) = out
    vt8 = np.ascontiguousarray(np.swapaxes(v8, -1, -2))
    return Fp8Inputs(q8=q8, k8=k8, vt8=vt8, q_descale=qd, k_descale=kd, v_descale=vd)
