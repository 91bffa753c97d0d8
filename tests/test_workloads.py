"""Seeded input generator: deterministic, correctly rounded, right shapes (CPU only)."""
import hashlib

import numpy as np
import pytest

from workloads import HBM_PROBES, WORKLOADS, f32_to_bf16_bits, make_inputs, make_random


def test_bf16_rounding_is_nearest_even():
    torch = pytest.importorskip("torch")
    x = np.random.default_rng(3).standard_normal(100000).astype(np.float32) * 37
    halfway = np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -(1.0 + 2 ** -8)], dtype=np.float32)
    x = np.concatenate([x, halfway])
    got = f32_to_bf16_bits(x)
    want = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(got, want)


def test_seeded_and_repeatable():
    w = WORKLOADS["tiny_causal_d64"]
    a, b = make_inputs(w), make_inputs(w)
    for x, y in ((a.q, b.q), (a.k, b.k), (a.v, b.v)):
        np.testing.assert_array_equal(x, y)
    h1 = hashlib.sha256(a.q.tobytes() + a.k.tobytes() + a.v.tobytes()).hexdigest()
    h2 = hashlib.sha256(b.q.tobytes() + b.k.tobytes() + b.v.tobytes()).hexdigest()
    assert h1 == h2
    assert a.q.shape == (1, 2, 256, 64) and a.q.dtype == np.uint16


def test_varlen_workload_masks():
    inp = make_inputs(WORKLOADS["varlen_n1024_d64"])
    assert inp.seqlens_k.dtype == np.int32 and inp.seqlens_k.shape == (8,)
    assert np.all((inp.seqlens_k >= 256) & (inp.seqlens_k <= 1024))
    np.testing.assert_array_equal(inp.q_start, [0, 64, 0, 0, 0, 64, 0, 0])


def test_stress_workload_q_std():
    w = WORKLOADS["causal_n16384_d128_stress"]
    g = np.random.Generator(np.random.PCG64(w.seed))
    q = g.standard_normal((1, 1, 4096, 128), dtype=np.float32)   # same first draws as the workload
    assert abs(float((2 * q).std()) - 2.0) < 0.02


def test_make_random_shapes():
    q, k, v = make_random(2, 3, 5, 7, 64, seed=1)
    assert q.shape == (2, 3, 5, 64) and k.shape == (2, 3, 7, 64) and v.dtype == np.uint16


def test_flops_formula():
    w = WORKLOADS["causal_n4096_d128"]
    assert w.flops() == 4 * 32 * 4096 * 4096 * 128 / 2
    assert WORKLOADS["noncausal_n4096_d128"].flops() == 4 * 32 * 4096 * 4096 * 128


def test_hbm_probes_sit_below_the_ridge():
    # counted flops per algorithmic byte below 2.5 PFLOP/s / 8 TB/s, inputs larger than the 256 MB cache
    for w in HBM_PROBES.values():
        assert w.flops() / w.algorithmic_bytes() < 2500.0 / 8.0
        assert 3 * 2 * w.B * w.H * w.N_k * w.d > 256 << 20


def test_fp8_inputs_are_deterministic_and_scaled():
    import numpy as np

    from oracle.fp8 import e4m3_decode
    from workloads import make_fp8

    a, b = make_fp8(1, 2, 30, 40, 64, seed=9), make_fp8(1, 2, 30, 40, 64, seed=9)
    for x, y in ((a.q8, b.q8), (a.k8, b.k8), (a.vt8, b.vt8)):
        np.testing.assert_array_equal(x, y)
    assert (a.q_descale, a.k_descale, a.v_descale) == (b.q_descale, b.k_descale, b.v_descale)
    assert not np.array_equal(make_fp8(1, 2, 30, 40, 64, seed=10).q8, a.q8)
    # each tensor's largest magnitude maps to 448 (the largest E4M3 value)
    for codes, ds in ((a.q8, a.q_descale), (a.k8, a.k_descale), (a.vt8, a.v_descale)):
        assert np.abs(e4m3_decode(codes)).max() == 448.0 and ds > 0
