"""Pins of the fp64 oracle against facts other than its own code (CPU only).

Each test fixes a result by something the oracle does not compute the same
way: a hand-worked example, a closed form, an invariant of the mathematics, a
brute-force loop, or a separate library routine. Together they fail on a
dropped scale, a wrong sign, a transposed operand, a wrong mask index, a
missing max subtraction or a wrong log-sum-exp.
"""
import json
import math
import os

import numpy as np
import pytest

from oracle import allowed_mask, attention, attention_online, bf16_bits_to_f64

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rnd(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


# ---------------------------------------------------------------- golden
@pytest.mark.parametrize("impl", ["two_pass", "online"])
def test_hand_worked_2x2(impl):
    """Closed-form 2x2 example (tests/golden/worked_2x2.json), every mask rule."""
    with open(os.path.join(GOLDEN, "worked_2x2.json"), encoding="utf-8") as f:
        fx = json.load(f)
    q = np.array(fx["Q"], float)[None, None]
    k = np.array(fx["K"], float)[None, None]
    v = np.array(fx["V"], float)[None, None]
    for case in fx["cases"]:
        kw = dict(causal=case["causal"], seqlens_k=np.array([case["kv_len"]]), q_start=np.array([case["q_start"]]))
        if impl == "two_pass":
            o, lse = attention(q, k, v, fx["scale"], **kw)
        else:
            o, lse = attention_online(q, k, v, fx["scale"], block_k=1, **kw)
        want_o = np.array(case["O"], float)
        want_l = np.array([-np.inf if x is None else x for x in case["LSE"]])
        np.testing.assert_allclose(o[0, 0], want_o, rtol=0, atol=1e-13, err_msg=case["name"])
        np.testing.assert_array_equal(np.isneginf(lse[0, 0]), np.isneginf(want_l))
        fin = np.isfinite(want_l)
        np.testing.assert_allclose(lse[0, 0][fin], want_l[fin], rtol=0, atol=1e-13, err_msg=case["name"])


def test_one_by_one():
    """1x1x1: softmax of a single score is 1, O = V, LSE = q*k*scale."""
    o, lse = attention(np.array([[[[3.0]]]]), np.array([[[[-2.0]]]]), np.array([[[[7.5]]]]), 0.25)
    assert o[0, 0, 0, 0] == 7.5
    assert lse[0, 0, 0] == -1.5


# ---------------------------------------------------------------- closed forms
@pytest.mark.parametrize("causal", [False, True])
def test_q_zero_gives_mean_of_allowed_v(causal):
    """Q = 0: every allowed score is 0, so O_i is the plain mean of the allowed V rows
    and LSE_i = ln(number of allowed keys)."""
    B, H, nq, nk, d = 2, 2, 9, 11, 5
    k, v = rnd((B, H, nk, d), 1), rnd((B, H, nk, d), 2)
    q = np.zeros((B, H, nq, d))
    seq = np.array([11, 6])
    qs = np.array([0, 3])
    o, lse = attention(q, k, v, 0.7, causal=causal, seqlens_k=seq, q_start=qs)
    for b in range(B):
        for h in range(H):
            for i in range(nq):
                hi = min(seq[b], i + 1) if causal else seq[b]
                if i < qs[b] or hi <= 0:
                    assert np.all(o[b, h, i] == 0) and np.isneginf(lse[b, h, i])
                    continue
                np.testing.assert_allclose(o[b, h, i], v[b, h, :hi].mean(axis=0), atol=1e-14)
                assert abs(lse[b, h, i] - math.log(hi)) < 1e-14


def test_scale_zero_equals_q_zero():
    q, k, v = rnd((1, 1, 6, 4), 3), rnd((1, 1, 6, 4), 4), rnd((1, 1, 6, 4), 5)
    o, lse = attention(q, k, v, 0.0, causal=True)
    o0, lse0 = attention(np.zeros_like(q), k, v, 1.0, causal=True)
    np.testing.assert_allclose(o, o0, atol=1e-15)
    np.testing.assert_allclose(lse, lse0, atol=1e-15)


@pytest.mark.parametrize("causal", [False, True])
def test_single_dominant_logit_selects_its_value_row(causal):
    """K rows are one-hot e_j; Q_i = a * e_{j*(i)}. Then S_ij = a*scale if j == j*(i) else 0,
    so O_i = (e^{a s} V_{j*} + sum_{j != j*} V_j) / (e^{a s} + n_i - 1) and
    LSE_i = a s + ln(1 + (n_i - 1) e^{-a s}); with a s = 125, O_i = V_{j*}."""
    nk = d = 8
    nq = 8
    rng = np.random.default_rng(7)
    k = np.eye(d)[None, None]
    v = rnd((1, 1, nk, d), 8)
    star = np.array([rng.integers(0, (i + 1) if causal else nk) for i in range(nq)])
    scale = 0.125
    for a in (24.0, 1000.0):
        q = np.zeros((1, 1, nq, d))
        q[0, 0, np.arange(nq), star] = a
        o, lse = attention(q, k, v, scale, causal=causal)
        z = a * scale
        for i in range(nq):
            n = (i + 1) if causal else nk
            others = [j for j in range(n) if j != star[i]]
            want = (math.exp(z) * v[0, 0, star[i]] + v[0, 0, others].sum(axis=0)) / (math.exp(z) + n - 1) \
                if z < 700 else v[0, 0, star[i]]
            np.testing.assert_allclose(o[0, 0, i], want, rtol=1e-12, atol=1e-12)
            want_l = z + math.log1p((n - 1) * math.exp(-z))
            assert abs(lse[0, 0, i] - want_l) < 1e-12 * max(1, z)


def test_causal_row_zero_is_v0():
    q, k, v = rnd((2, 3, 5, 4), 9), rnd((2, 3, 5, 4), 10), rnd((2, 3, 5, 4), 11)
    o, lse = attention(q, k, v, 0.3, causal=True)
    np.testing.assert_array_equal(o[:, :, 0], v[:, :, 0])
    np.testing.assert_allclose(lse[:, :, 0], 0.3 * np.einsum("bhd,bhd->bh", q[:, :, 0], k[:, :, 0]), atol=1e-15)


# ---------------------------------------------------------------- invariants
def test_probs_are_a_masked_distribution():
    B, H, nq, nk, d = 2, 2, 13, 17, 6
    q, k, v = rnd((B, H, nq, d), 12, 3), rnd((B, H, nk, d), 13), rnd((B, H, nk, d), 14)
    seq, qs = np.array([17, 5]), np.array([4, 0])
    _, lse, p = attention(q, k, v, 0.4, causal=True, seqlens_k=seq, q_start=qs, return_probs=True)
    assert np.all(p >= 0)
    for b in range(B):
        ok = allowed_mask(nq, nk, True, seq[b], qs[b])
        assert np.all(p[b][:, ~ok] == 0)
        live = ok.any(axis=1)
        np.testing.assert_allclose(p[b][:, live].sum(axis=-1), 1.0, atol=1e-14)
        assert np.all(p[b][:, ~live] == 0)
        assert np.all(np.isneginf(lse[b][:, ~live]))


def test_constant_v_gives_constant_o():
    q, k = rnd((1, 2, 7, 5), 15, 2), rnd((1, 2, 9, 5), 16)
    v = np.full((1, 2, 9, 5), -1.25)
    o, _ = attention(q, k, v, 0.5, causal=False, seqlens_k=np.array([6]))
    np.testing.assert_allclose(o, -1.25, atol=1e-15)


def test_identity_v_exposes_probs():
    nq, nk, d = 6, 5, 8
    q, k = rnd((1, 1, nq, d), 17), rnd((1, 1, nk, d), 18)
    v = np.zeros((1, 1, nk, d))
    v[0, 0, :, :nk] = np.eye(nk)
    o, _, p = attention(q, k, v, 0.9, causal=True, return_probs=True)
    np.testing.assert_allclose(o[0, 0, :, :nk], p[0, 0], atol=1e-15)
    # and P row i is the softmax of the visible scores, computed independently here
    s = (q[0, 0] @ k[0, 0].T) * 0.9
    for i in range(nq):
        e = np.exp(s[i, :i + 1] - s[i, :i + 1].max())
        np.testing.assert_allclose(p[0, 0, i, :i + 1], e / e.sum(), atol=1e-15)


def test_shift_of_all_logits_moves_lse_not_o():
    """Append a column of ones to K and alpha to Q: every score moves by alpha*scale."""
    q, k, v = rnd((1, 2, 5, 4), 19), rnd((1, 2, 8, 4), 20), rnd((1, 2, 8, 4), 21)
    alpha, scale = 3.5, 0.6
    q2 = np.concatenate([q, np.full((1, 2, 5, 1), alpha)], axis=-1)
    k2 = np.concatenate([k, np.ones((1, 2, 8, 1))], axis=-1)
    o, lse = attention(q, k, v, scale, causal=True)
    o2, lse2 = attention(q2, k2, v, scale, causal=True)
    np.testing.assert_allclose(o2, o, atol=1e-14)
    np.testing.assert_allclose(lse2, lse + alpha * scale, atol=1e-13)


def test_key_permutation_invariance():
    q, k, v = rnd((2, 1, 6, 4), 22), rnd((2, 1, 10, 4), 23), rnd((2, 1, 10, 4), 24)
    perm = np.random.default_rng(25).permutation(10)
    o, lse = attention(q, k, v, 0.5)
    o2, lse2 = attention(q, k[:, :, perm], v[:, :, perm], 0.5)
    np.testing.assert_allclose(o2, o, atol=1e-14)
    np.testing.assert_allclose(lse2, lse, atol=1e-14)


def test_padding_contents_are_ignored():
    q, k, v = rnd((1, 1, 4, 3), 26), rnd((1, 1, 6, 3), 27), rnd((1, 1, 6, 3), 28)
    k2, v2 = k.copy(), v.copy()
    k2[0, 0, 4:] = np.nan
    v2[0, 0, 4:] = np.inf
    for impl in (attention, attention_online):
        o, lse = impl(q, k, v, 0.5, seqlens_k=np.array([4]))
        o2, lse2 = impl(q, k2, v2, 0.5, seqlens_k=np.array([4]))
        np.testing.assert_array_equal(o2, o)
        np.testing.assert_array_equal(lse2, lse)


def test_no_keys_and_no_rows():
    q = rnd((1, 2, 3, 4), 29)
    e = np.zeros((1, 2, 0, 4))
    o, lse = attention(q, e, e, 1.0)
    assert np.all(o == 0) and np.all(np.isneginf(lse))
    o, lse = attention(np.zeros((1, 2, 0, 4)), rnd((1, 2, 3, 4), 30), rnd((1, 2, 3, 4), 31), 1.0)
    assert o.shape == (1, 2, 0, 4) and lse.shape == (1, 2, 0)


def test_rows_subset_matches_full():
    q, k, v = rnd((1, 2, 40, 8), 32), rnd((1, 2, 40, 8), 33), rnd((1, 2, 40, 8), 34)
    rows = [0, 1, 17, 39]
    o, lse = attention(q, k, v, 0.3, causal=True, row_block=7)
    os_, lses = attention(q, k, v, 0.3, causal=True, rows=rows)
    np.testing.assert_array_equal(os_, o[:, :, rows])
    np.testing.assert_array_equal(lses, lse[:, :, rows])


# ---------------------------------------------------------------- brute force
def test_allowed_mask_matches_loops():
    for causal in (False, True):
        for kv, qs in ((None, None), (7, 0), (0, 0), (20, 3), (-5, 99), (3, -1)):
            ok = allowed_mask(9, 12, causal, kv, qs)
            kvc = 12 if kv is None else min(max(kv, 0), 12)
            qsc = 0 if qs is None else min(max(qs, 0), 9)
            for i in range(9):
                for j in range(12):
                    want = j < kvc and i >= qsc and (not causal or j <= i)
                    assert ok[i, j] == want


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("T", [1, 3, 7, 16, 64])
def test_online_recurrence_equals_two_pass(causal, T):
    """The pages state the tiled recurrence gives the full-matrix result exactly."""
    B, H, nq, nk, d = 3, 2, 21, 37, 8
    q, k, v = rnd((B, H, nq, d), 40 + T, 2.0), rnd((B, H, nk, d), 41), rnd((B, H, nk, d), 42)
    seq = np.array([37, 0, 19])
    qs = np.array([0, 0, 5])
    o, lse = attention(q, k, v, 0.45, causal=causal, seqlens_k=seq, q_start=qs)
    o2, lse2 = attention_online(q, k, v, 0.45, causal=causal, seqlens_k=seq, q_start=qs, block_k=min(T, nk))
    np.testing.assert_allclose(o2, o, rtol=1e-12, atol=1e-13)
    fin = np.isfinite(lse)
    np.testing.assert_array_equal(np.isfinite(lse2), fin)
    np.testing.assert_allclose(lse2[fin], lse[fin], rtol=1e-12, atol=1e-12)


def test_bf16_expansion_is_exact():
    bits = np.array([0x3F80, 0xBF80, 0x0000, 0x8000, 0x7F80, 0xFF80, 0x4049, 0x0001], dtype=np.uint16)
    want = np.array([1.0, -1.0, 0.0, -0.0, np.inf, -np.inf, 3.140625, 2.0 ** -133])
    got = bf16_bits_to_f64(bits)
    np.testing.assert_array_equal(got, want)


# ---------------------------------------------------------------- library cross-check
def test_torch_sdpa_cpu_fp64_cross_check():
    """torch's CPU SDPA (math path) in float64 with the same boolean mask."""
    torch = pytest.importorskip("torch")
    import torch.nn.functional as F

    B, H, nq, nk, d = 2, 3, 19, 23, 16
    q, k, v = rnd((B, H, nq, d), 50, 2), rnd((B, H, nk, d), 51), rnd((B, H, nk, d), 52)
    seq, qs = np.array([23, 9]), np.array([0, 4])
    o, lse = attention(q, k, v, 0.3, causal=True, seqlens_k=seq, q_start=qs)
    mask = np.stack([allowed_mask(nq, nk, True, seq[b], qs[b]) for b in range(B)])[:, None]
    got = F.scaled_dot_product_attention(torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v),
                                         attn_mask=torch.from_numpy(mask), scale=0.3).numpy()
    live = mask[:, 0].any(axis=-1)
    for h in range(H):
        np.testing.assert_allclose(o[:, h][live], got[:, h][live], rtol=1e-12, atol=1e-12)
    if np.all(np.isfinite(got)):   # torch's math path is NaN-safe: fully masked rows give 0
        for h in range(H):
            np.testing.assert_array_equal(got[:, h][~live], 0.0)
            np.testing.assert_array_equal(o[:, h][~live], 0.0)


# ---------------------------------------------------------------- bottom-right causal (causal = 2)
def test_bottom_right_mask_brute_force():
    for n_q, n_k in [(3, 7), (7, 3), (5, 5), (1, 6)]:
        ok = allowed_mask(n_q, n_k, 2)
        for i in range(n_q):
            for j in range(n_k):
                assert ok[i, j] == (j - (n_k - n_q) <= i), (n_q, n_k, i, j)


def test_bottom_right_single_query_sees_every_key():
    """One query row at the end of the key sequence (decoding against a cache):
    bottom-right causal is plain attention over all keys."""
    q, k, v = rnd((2, 3, 1, 8), 51), rnd((2, 3, 9, 8), 52), rnd((2, 3, 9, 8), 53)
    o2, l2 = attention(q, k, v, 0.3, 2)
    o0, l0 = attention(q, k, v, 0.3, False)
    np.testing.assert_allclose(o2, o0, atol=1e-14)
    np.testing.assert_allclose(l2, l0, atol=1e-14)
    o1, _ = attention(q, k, v, 0.3, True)          # top-left: row 0 sees only key 0
    np.testing.assert_allclose(o1[:, :, 0], v[:, :, 0], atol=1e-14)


@pytest.mark.parametrize("n_q,n_k", [(4, 9), (9, 4)])
def test_bottom_right_prefix_mean_closed_form(n_q, n_k):
    """Q = 0: row i averages V over keys 0 .. i + n_k - n_q (no key: O = 0, LSE = -inf)."""
    q = np.zeros((1, 1, n_q, 3))
    k, v = rnd((1, 1, n_k, 3), 54), rnd((1, 1, n_k, 3), 55)
    o, lse = attention(q, k, v, 1.0, 2)
    oo, lo = attention_online(q, k, v, 1.0, 2, block_k=2)
    for i in range(n_q):
        last = i + n_k - n_q
        if last < 0:
            assert np.all(o[0, 0, i] == 0) and np.isneginf(lse[0, 0, i])
        else:
            np.testing.assert_allclose(o[0, 0, i], v[0, 0, :last + 1].mean(axis=0), atol=1e-14)
            assert abs(lse[0, 0, i] - math.log(last + 1)) < 1e-14
    np.testing.assert_allclose(oo, o, atol=1e-13)


def test_bottom_right_torch_cross_check():
    torch = pytest.importorskip("torch")
    try:
        from torch.nn.attention.bias import causal_lower_right
    except ImportError:
        pytest.skip("torch has no bottom-right causal bias")
    q, k, v = rnd((1, 2, 5, 6), 56), rnd((1, 2, 8, 6), 57), rnd((1, 2, 8, 6), 58)
    tq, tk, tv = (torch.tensor(x) for x in (q, k, v))
    want = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=causal_lower_right(5, 8),
                                                            scale=0.4).numpy()
    o, _ = attention(q, k, v, 0.4, 2)
    np.testing.assert_allclose(o, want, atol=1e-12)


# ---------------------------------------------------------------- boolean attn_mask (True = may attend)
def softmax_loops(q, k, v, scale, allowed):
    """Pure-Python loops over one head: the definition written out entry by entry."""
    n_q, n_k = allowed.shape
    out = np.zeros((n_q, v.shape[1]))
    lse = np.full(n_q, -np.inf)
    for i in range(n_q):
        sc = [sum(q[i, t] * k[j, t] for t in range(q.shape[1])) * scale for j in range(n_k) if allowed[i, j]]
        idx = [j for j in range(n_k) if allowed[i, j]]
        if not idx:
            continue
        m = max(sc)
        e = [math.exp(x - m) for x in sc]
        tot = sum(e)
        for w, j in zip(e, idx):
            out[i] += w / tot * v[j]
        lse[i] = m + math.log(tot)
    return out, lse


def test_dense_mask_brute_force_loops():
    rng = np.random.default_rng(71)
    q, k, v = rnd((2, 2, 6, 3), 72), rnd((2, 2, 7, 3), 73), rnd((2, 2, 7, 3), 74)
    mask = rng.random((2, 1, 6, 7)) < 0.6          # broadcast over heads
    mask[1, 0, 2] = False                           # one fully masked row
    o, lse = attention(q, k, v, 0.5, False, attn_mask=mask)
    for b in range(2):
        for h in range(2):
            wo, wl = softmax_loops(q[b, h], k[b, h], v[b, h], 0.5, mask[b, 0])
            np.testing.assert_allclose(o[b, h], wo, atol=1e-13)
            np.testing.assert_allclose(lse[b, h], wl, atol=1e-13)
    assert np.all(o[1, :, 2] == 0) and np.all(np.isneginf(lse[1, :, 2]))


def test_dense_mask_reproduces_the_rule_masks():
    q, k, v = rnd((2, 2, 9, 4), 75), rnd((2, 2, 9, 4), 76), rnd((2, 2, 9, 4), 77)
    sl, qs = np.array([9, 5]), np.array([0, 3])
    want_o, want_l = attention(q, k, v, 0.6, True, seqlens_k=sl, q_start=qs)
    m = np.zeros((2, 1, 9, 9), bool)
    for b in range(2):
        m[b, 0] = allowed_mask(9, 9, True, sl[b], qs[b])
    o, lse = attention(q, k, v, 0.6, False, attn_mask=m)
    np.testing.assert_allclose(o, want_o, atol=1e-14)
    np.testing.assert_array_equal(np.isneginf(lse), np.isneginf(want_l))
    np.testing.assert_allclose(lse[~np.isneginf(lse)], want_l[~np.isneginf(want_l)], atol=1e-14)
    # the mask intersects the rules: all-True changes nothing
    o2, _ = attention(q, k, v, 0.6, True, seqlens_k=sl, q_start=qs, attn_mask=np.ones((1, 1, 9, 9), bool))
    np.testing.assert_array_equal(o2, want_o)


def test_dense_mask_torch_cross_check():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(78)
    q, k, v = rnd((2, 3, 7, 5), 79), rnd((2, 3, 10, 5), 80), rnd((2, 3, 10, 5), 81)
    mask = rng.random((2, 3, 7, 10)) < 0.5
    mask[..., 0] = True                              # no fully masked row (torch gives NaN there)
    want = torch.nn.functional.scaled_dot_product_attention(
        torch.tensor(q), torch.tensor(k), torch.tensor(v), attn_mask=torch.tensor(mask), scale=0.35).numpy()
    o, _ = attention(q, k, v, 0.35, False, attn_mask=mask)
    np.testing.assert_allclose(o, want, atol=1e-12)


def test_block_mask_expansion_brute_force():
    from oracle import expand_block_mask
    rng = np.random.default_rng(101)
    bm = rng.random((2, 3, 3, 5)) < 0.5
    m = expand_block_mask(bm, 7, 9, 3, 2)
    assert m.shape == (2, 3, 7, 9)
    for b in range(2):
        for h in range(3):
            for i in range(7):
                for j in range(9):
                    assert m[b, h, i, j] == bm[b, h, i // 3, j // 2]
