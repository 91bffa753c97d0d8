"""Pins of the FP8 forward oracle (CPU only).

``e4m3_decode`` is fixed by the values the OCP E4M3 format defines and by
torch's float8_e4m3fn as a separate library; ``attention_fp8`` by a pure-Python
brute force on tiny inputs (which also fixes the transposed V layout and where
each descale applies), closed forms and invariances.
"""
import math

import numpy as np
import pytest

from oracle.fp8 import attention_fp8, e4m3_decode
from workloads import make_fp8


@pytest.mark.parametrize("code,value", [
    (0x38, 1.0), (0x40, 2.0), (0x3C, 1.5), (0x30, 0.5), (0x7E, 448.0), (0x08, 2.0 ** -6),
    (0x01, 2.0 ** -9), (0x07, 7 * 2.0 ** -9), (0x00, 0.0), (0xB8, -1.0), (0xFE, -448.0), (0x77, 240.0),
])
def test_decode_defining_values(code, value):
    assert e4m3_decode(np.array([code], dtype=np.uint8))[0] == value


def test_decode_sign_and_nan():
    z = e4m3_decode(np.array([0x80], dtype=np.uint8))[0]
    assert z == 0.0 and math.copysign(1.0, z) < 0
    assert np.isnan(e4m3_decode(np.array([0x7F, 0xFF], dtype=np.uint8))).all()
    # every other code with exponent field 15 is a finite number (no infinities)
    assert np.isfinite(e4m3_decode(np.arange(0x78, 0x7F, dtype=np.uint8))).all()


def test_decode_monotone():
    v = e4m3_decode(np.arange(0, 0x7F, dtype=np.uint8))
    assert np.all(np.diff(v) > 0)


def test_decode_matches_torch_float8():
    torch = pytest.importorskip("torch")
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = e4m3_decode(codes)
    np.testing.assert_array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    np.testing.assert_array_equal(got[ok], ref[ok])


def _brute(x, scale, causal):
    """Pure-Python attention over the decoded codes, one row at a time."""
    def dec(c):
        c = int(c)
        s, e, m = c >> 7, (c >> 3) & 15, c & 7
        mag = (1 + m / 8) * 2.0 ** (e - 7) if e else (m / 8) * 2.0 ** -6
        return -mag if s else mag
    B, H, n_q, d = x.q8.shape
    n_k = x.k8.shape[2]
    o = np.zeros((B, H, n_q, d))
    lse = np.full((B, H, n_q), -np.inf)
    for b in range(B):
        for h in range(H):
            for i in range(n_q):
                keys = [j for j in range(n_k) if not causal or j <= i]
                if not keys:
                    continue
                s = [sum(dec(x.q8[b, h, i, t]) * x.q_descale * dec(x.k8[b, h, j, t]) * x.k_descale
                         for t in range(d)) * scale for j in keys]
                mx = max(s)
                p = [math.exp(v - mx) for v in s]
                tot = sum(p)
                lse[b, h, i] = mx + math.log(tot)
                for c in range(d):
                    o[b, h, i, c] = sum(pj * dec(x.vt8[b, h, c, j]) * x.v_descale for pj, j in zip(p, keys)) / tot
    return o, lse


@pytest.mark.parametrize("causal", [False, True])
def test_brute_force_tiny(causal):
    x = make_fp8(1, 2, 5, 7, 4, seed=3, sigma=(2.0, 2.0, 1.0))
    o, lse = attention_fp8(x.q8, x.k8, x.vt8, 0.6, x.q_descale, x.k_descale, x.v_descale, causal)
    bo, bl = _brute(x, 0.6, causal)
    np.testing.assert_allclose(o, bo, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse, bl, rtol=1e-12, atol=1e-13)


def test_zero_queries_average_values():
    """Q = 0: every visible key has the same weight, O is the mean of the V rows."""
    x = make_fp8(1, 1, 6, 9, 8, seed=4)
    x.q8[:] = 0
    o, lse = attention_fp8(x.q8, x.k8, x.vt8, 0.3, x.q_descale, x.k_descale, x.v_descale, True)
    v = e4m3_decode(x.vt8[0, 0]).T * x.v_descale          # [N_k, d]
    for i in range(6):
        np.testing.assert_allclose(o[0, 0, i], v[: i + 1].mean(axis=0), rtol=1e-12, atol=1e-15)
        np.testing.assert_allclose(lse[0, 0, i], math.log(i + 1), rtol=1e-12)


def test_equal_value_rows():
    x = make_fp8(1, 1, 5, 6, 8, seed=5)
    x.vt8[:] = x.vt8[:, :, :, :1]                             # every key carries key 0's V
    o, _ = attention_fp8(x.q8, x.k8, x.vt8, 0.5, x.q_descale, x.k_descale, x.v_descale, False)
    want = e4m3_decode(x.vt8[0, 0, :, 0]) * x.v_descale
    np.testing.assert_allclose(o[0, 0], np.broadcast_to(want, (5, 8)), rtol=1e-12, atol=1e-15)


def test_descale_invariances():
    x = make_fp8(1, 2, 7, 9, 8, seed=6)
    base_o, base_l = attention_fp8(x.q8, x.k8, x.vt8, 0.4, x.q_descale, x.k_descale, x.v_descale, True)
    # the scores depend on q_descale * k_descale * scale only
    o2, l2 = attention_fp8(x.q8, x.k8, x.vt8, 0.2, 4 * x.q_descale, 0.5 * x.k_descale, x.v_descale, True)
    np.testing.assert_allclose(o2, base_o, rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(l2, base_l, rtol=1e-12)
    # O is linear in v_descale, LSE does not depend on it
    o3, l3 = attention_fp8(x.q8, x.k8, x.vt8, 0.4, x.q_descale, x.k_descale, 3 * x.v_descale, True)
    np.testing.assert_allclose(o3, 3 * base_o, rtol=1e-12, atol=1e-15)
    np.testing.assert_array_equal(l3, base_l)


def test_generator_codes_in_range():
    x = make_fp8(2, 2, 33, 40, 16, seed=7)
    for c in (x.q8, x.k8, x.vt8):
        assert c.dtype == np.uint8 and not np.isnan(e4m3_decode(c)).any()
        assert np.abs(e4m3_decode(c)).max() == 448.0
    assert x.vt8.shape == (2, 2, 16, 40)
