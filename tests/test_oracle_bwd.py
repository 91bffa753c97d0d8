"""Pins of the fp64 backward oracle (CPU only).

Each test fixes the gradients by something ``attention_bwd`` does not compute
the same way: finite differences of the forward oracle, invariants of the
mathematics, a closed form, or torch's autograd as a separate library.
"""
import numpy as np
import pytest

from oracle import attention, attention_bwd, check_grads

CASES = [
    # n_q, n_k, d, causal, seqlens_k, q_start
    (5, 7, 4, False, None, None),
    (6, 6, 3, True, None, None),
    (7, 5, 4, True, [4, 5], [0, 2]),
    (4, 6, 2, False, [3, 0], [1, 0]),
]


def rnd(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


def loss(q, k, v, g, scale, causal, sl, qs):
    o, _ = attention(q, k, v, scale, causal, seqlens_k=sl, q_start=qs)
    return float((o * g).sum())


@pytest.mark.parametrize("case", CASES)
def test_finite_differences(case):
    """Central differences of <dO, O(Q, K, V)> through the forward oracle."""
    n_q, n_k, d, causal, sl, qs = case
    B = 2 if sl is not None else 1
    sl = None if sl is None else np.array(sl)
    qs = None if qs is None else np.array(qs)
    q, k, v = rnd((B, 2, n_q, d), 1), rnd((B, 2, n_k, d), 2), rnd((B, 2, n_k, d), 3)
    g = rnd((B, 2, n_q, d), 4)
    scale = 0.7
    dq, dk, dv = attention_bwd(q, k, v, g, scale, causal, sl, qs)
    eps = 1e-6
    for name, x, grad in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        num = np.zeros_like(x)
        it = np.nditer(x, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            xp, xm = x.copy(), x.copy()
            xp[idx] += eps
            xm[idx] -= eps
            args = {"q": q, "k": k, "v": v}
            args[name] = xp
            lp = loss(args["q"], args["k"], args["v"], g, scale, causal, sl, qs)
            args[name] = xm
            lm = loss(args["q"], args["k"], args["v"], g, scale, causal, sl, qs)
            num[idx] = (lp - lm) / (2 * eps)
        np.testing.assert_allclose(grad, num, rtol=1e-6, atol=1e-7, err_msg=f"d{name}")


@pytest.mark.parametrize("causal", [False, True])
def test_dk_sums_to_zero_over_keys(causal):
    """Adding one vector to every key shifts each row's scores by a constant,
    which the softmax ignores: the dK rows of a head sum to zero."""
    q, k, v, g = rnd((1, 3, 9, 5), 5), rnd((1, 3, 11, 5), 6), rnd((1, 3, 11, 5), 7), rnd((1, 3, 9, 5), 8)
    _, dk, _ = attention_bwd(q, k, v, g, 0.4, causal, np.array([8]), np.array([2]))
    np.testing.assert_allclose(dk.sum(axis=2), 0.0, atol=1e-12)
    assert np.abs(dk).max() > 1e-3


def test_zero_upstream_gradient():
    q, k, v = rnd((1, 2, 6, 4), 9), rnd((1, 2, 6, 4), 10), rnd((1, 2, 6, 4), 11)
    for t in attention_bwd(q, k, v, np.zeros_like(q), 0.5, True):
        assert np.all(t == 0)


def test_equal_value_rows_give_no_score_gradient():
    """V with equal rows makes O independent of the probabilities: dQ = dK = 0."""
    q, k = rnd((1, 2, 7, 4), 12), rnd((1, 2, 9, 4), 13)
    v = np.broadcast_to(rnd((1, 2, 1, 4), 14), (1, 2, 9, 4)).copy()
    g = rnd((1, 2, 7, 4), 15)
    dq, dk, dv = attention_bwd(q, k, v, g, 0.8, False)
    np.testing.assert_allclose(dq, 0.0, atol=1e-12)
    np.testing.assert_allclose(dk, 0.0, atol=1e-12)
    assert np.abs(dv).max() > 1e-3


@pytest.mark.parametrize("causal", [False, True])
def test_uniform_probabilities_closed_form(causal):
    """Q = 0: every row spreads its weight evenly over the keys it sees, so
    dV_j = sum over the rows i that see key j of dO_i / n_i, with n_i keys seen."""
    n_q, n_k, d = 6, 8, 3
    q = np.zeros((1, 1, n_q, d))
    k, v, g = rnd((1, 1, n_k, d), 16), rnd((1, 1, n_k, d), 17), rnd((1, 1, n_q, d), 18)
    kv, qs = 7, 1
    _, _, dv = attention_bwd(q, k, v, g, 1.0, causal, np.array([kv]), np.array([qs]))
    want = np.zeros((n_k, d))
    for i in range(n_q):
        seen = [j for j in range(n_k) if j < kv and i >= qs and (not causal or j <= i)]
        for j in seen:
            want[j] += g[0, 0, i] / len(seen)
    np.testing.assert_allclose(dv[0, 0], want, atol=1e-12)


def test_fully_masked_rows_pass_no_gradient():
    q, k, v, g = rnd((1, 1, 5, 4), 19), rnd((1, 1, 5, 4), 20), rnd((1, 1, 5, 4), 21), rnd((1, 1, 5, 4), 22)
    dq, dk, dv = attention_bwd(q, k, v, g, 0.5, False, q_start=np.array([3]))
    assert np.all(dq[0, 0, :3] == 0)
    g2 = g.copy()
    g2[0, 0, :3] = 1e3   # the masked rows' upstream gradient must not matter
    dq2, dk2, dv2 = attention_bwd(q, k, v, g2, 0.5, False, q_start=np.array([3]))
    np.testing.assert_array_equal(dk, dk2)
    np.testing.assert_array_equal(dv, dv2)


@pytest.mark.parametrize("causal", [False, True])
def test_torch_autograd_cross_check(causal):
    torch = pytest.importorskip("torch")
    B, H, n_q, n_k, d = 2, 2, 9, 9, 6
    q, k, v, g = rnd((B, H, n_q, d), 23), rnd((B, H, n_k, d), 24), rnd((B, H, n_k, d), 25), rnd((B, H, n_q, d), 26)
    sl = np.array([9, 6])
    scale = 0.45
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    j = torch.arange(n_k)
    i = torch.arange(n_q)
    allowed = (j[None, None, None, :] < torch.tensor(sl)[:, None, None, None]).expand(B, H, n_q, n_k)
    if causal:
        allowed = allowed & (j[None, :] <= i[:, None])
    s = (tq @ tk.transpose(-1, -2)) * scale
    s = s.masked_fill(~allowed, float("-inf"))
    o = torch.softmax(s, dim=-1) @ tv
    o.backward(torch.tensor(g))
    dq, dk, dv = attention_bwd(q, k, v, g, scale, causal, sl)
    np.testing.assert_allclose(dq, tq.grad.numpy(), atol=1e-12)
    np.testing.assert_allclose(dk, tk.grad.numpy(), atol=1e-12)
    np.testing.assert_allclose(dv, tv.grad.numpy(), atol=1e-12)


def test_grad_checker_bars():
    r = {"dq": np.ones((2, 3)), "dk": np.zeros((2, 3)), "dv": np.full((2, 3), 5.0)}
    assert check_grads({k: v.copy() for k, v in r.items()}, r).ok
    bad = {k: v.copy() for k, v in r.items()}
    bad["dv"][0, 0] += 0.2       # above 2e-2 * 5
    assert not check_grads(bad, r).ok
    bad = {k: v.copy() for k, v in r.items()}
    bad["dq"][:] += 0.011        # mean above 1 % of mean |dq| = 1
    assert not check_grads(bad, r).ok
    ok = {k: v.copy() for k, v in r.items()}
    ok["dq"][:] += 0.009
    assert check_grads(ok, r).ok
    bad = {k: v.copy() for k, v in r.items()}
    bad["dk"][0, 0] = 1e-4       # the reference is all zeros: only the 1e-6 floor remains
    assert not check_grads(bad, r).ok
    bad = {k: v.copy() for k, v in r.items()}
    bad["dq"][1, 2] = np.nan
    assert not check_grads(bad, r).ok


def test_finite_differences_bottom_right():
    n_q, n_k, d = 4, 7, 3
    q, k, v, g = rnd((1, 1, n_q, d), 61), rnd((1, 1, n_k, d), 62), rnd((1, 1, n_k, d), 63), rnd((1, 1, n_q, d), 64)
    dq, dk, dv = attention_bwd(q, k, v, g, 0.6, 2)
    eps = 1e-6
    for name, x, grad in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        num = np.zeros_like(x)
        it = np.nditer(x, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            args = {"q": q, "k": k, "v": v}
            xp, xm = x.copy(), x.copy()
            xp[idx] += eps
            xm[idx] -= eps
            args[name] = xp
            lp = loss(args["q"], args["k"], args["v"], g, 0.6, 2, None, None)
            args[name] = xm
            lm = loss(args["q"], args["k"], args["v"], g, 0.6, 2, None, None)
            num[idx] = (lp - lm) / (2 * eps)
        np.testing.assert_allclose(grad, num, rtol=1e-6, atol=1e-7, err_msg=f"d{name}")


def test_finite_differences_dense_mask():
    n_q, n_k, d = 5, 6, 3
    q, k, v, g = rnd((1, 2, n_q, d), 85), rnd((1, 2, n_k, d), 86), rnd((1, 2, n_k, d), 87), rnd((1, 2, n_q, d), 88)
    mask = np.random.default_rng(89).random((1, 2, n_q, n_k)) < 0.5
    mask[0, 1, 3] = False
    dq, dk, dv = attention_bwd(q, k, v, g, 0.6, False, attn_mask=mask)

    def lossm(q_, k_, v_):
        o, _ = attention(q_, k_, v_, 0.6, False, attn_mask=mask)
        return float((o * g).sum())
    eps = 1e-6
    for name, x, grad in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        num = np.zeros_like(x)
        it = np.nditer(x, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            args = {"q": q, "k": k, "v": v}
            xp, xm = x.copy(), x.copy()
            xp[idx] += eps
            xm[idx] -= eps
            args[name] = xp
            lp = lossm(args["q"], args["k"], args["v"])
            args[name] = xm
            lm = lossm(args["q"], args["k"], args["v"])
            num[idx] = (lp - lm) / (2 * eps)
        np.testing.assert_allclose(grad, num, rtol=1e-6, atol=1e-7, err_msg=f"d{name}")
    assert np.all(dq[0, 1, 3] == 0)
