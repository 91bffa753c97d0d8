"""The tolerance checker rejects what it must (CPU only)."""
import numpy as np

from oracle.checker import check, LSE_MAX_ABS, O_MAX_ABS


def ref():
    rng = np.random.default_rng(0)
    o = rng.standard_normal((2, 3, 16, 8)) * 0.1
    lse = rng.standard_normal((2, 3, 16)) + 5
    o[0, 1, 3] = 0.0
    lse[0, 1, 3] = -np.inf        # one fully masked row
    return o, lse


def test_exact_copy_passes():
    o, lse = ref()
    r = check(o.copy(), o, lse.copy(), lse)
    assert r.ok, str(r)


def test_within_tolerance_passes():
    o, lse = ref()
    o2 = o + 0.5 * O_MAX_ABS * np.sign(np.random.default_rng(1).standard_normal(o.shape)) * 0.002 / O_MAX_ABS
    o2[0, 1, 3] = 0.0
    r = check(o2, o, lse + 0.5 * LSE_MAX_ABS, lse)
    assert r.ok, str(r)


def test_nan_in_o_fails():
    o, lse = ref()
    o2 = o.copy()
    o2[1, 2, 5, 4] = np.nan
    assert not check(o2, o, lse, lse).ok


def test_max_abs_fails():
    o, lse = ref()
    o2 = o.copy()
    o2[1, 0, 0, 0] += 1.5 * O_MAX_ABS
    assert not check(o2, o, lse, lse).ok


def test_mean_abs_fails():
    o, lse = ref()
    o2 = o + 0.003
    o2[0, 1, 3] = 0.0
    r = check(o2, o, lse, lse)
    assert not r.ok and "mean" in str(r)


def test_masked_row_must_be_zero():
    o, lse = ref()
    o2 = o.copy()
    o2[0, 1, 3, 0] = 1e-6
    assert not check(o2, o, lse, lse).ok


def test_masked_row_lse_must_be_minus_inf():
    o, lse = ref()
    l2 = lse.copy()
    l2[0, 1, 3] = -1e30
    assert not check(o, o, l2, lse).ok


def test_lse_nan_or_out_of_band_fails():
    o, lse = ref()
    l2 = lse.copy()
    l2[1, 1, 1] = np.nan
    assert not check(o, o, l2, lse).ok
    l3 = lse.copy()
    l3[1, 1, 1] += 2 * LSE_MAX_ABS
    assert not check(o, o, l3, lse).ok


def test_spurious_minus_inf_fails():
    o, lse = ref()
    l2 = lse.copy()
    l2[1, 1, 2] = -np.inf
    assert not check(o, o, l2, lse).ok
