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


def test_merge_equals_whole_check():
    # slice-by-slice checking with the mean bar left to merge() gives the same
    # verdict and statistics as checking the whole output at once
    from oracle.checker import merge
    o, lse = ref()
    rng = np.random.default_rng(7)
    o2 = o + rng.uniform(-1.5e-3, 3.0e-3, o.shape)
    o2[0, 1, 3] = 0.0
    whole = check(o2, o, lse, lse)
    parts = [check(o2[b, h], o[b, h], lse[b, h], lse[b, h], mean_bar=False) for b in range(2) for h in range(3)]
    m = merge(parts)
    assert m.ok == whole.ok
    assert np.isclose(m.o_mean_abs, whole.o_mean_abs) and m.o_max_abs == whole.o_max_abs
    assert m.lse_max_abs == whole.lse_max_abs


def test_merge_applies_mean_bar_over_all_slices():
    # every slice alone would pass a per-slice max bar; the merged mean is over
    # the bar, so the merged verdict fails even though no slice tested its mean
    from oracle.checker import O_MEAN_ABS, merge
    o, lse = ref()
    o2 = o + 1.5 * O_MEAN_ABS
    o2[0, 1, 3] = 0.0
    parts = [check(o2[b, h], o[b, h], lse[b, h], lse[b, h], mean_bar=False) for b in range(2) for h in range(3)]
    assert all(p.ok for p in parts)
    m = merge(parts)
    assert not m.ok and any("mean" in r for r in m.reasons)
    # a structural failure in one slice survives the merge
    o3 = o.copy()
    o3[1, 2, 0, 0] = np.nan
    parts = [check(o3[b, h], o[b, h], lse[b, h], lse[b, h], mean_bar=False) for b in range(2) for h in range(3)]
    assert not merge(parts).ok
