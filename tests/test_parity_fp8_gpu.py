"""GPU parity of attn_fwd_fp8 against the fp64 FP8 oracle.

The kernel rounds 2^8 * P to E4M3 before the second product; the oracle is
attention over the dequantized inputs without that rounding. The bars follow
from the rounding (round to nearest even, 3 mantissa bits):
  * elementwise, the worst case: each p_j is off by at most 2^-4 p_j (normal
    range) or 2^-18 (half the subnormal spacing 2^-9, divided by 2^8), so
    |O - O_ref| <= 2^-4 A + 2^-18 n max|v| + 2^-8 |O_ref| (+ fp32 rounding),
    with A = sum_j p_j |v_j| / sum_j p_j and n the visible keys; the last term
    is the bf16 rounding of the output;
  * over all elements, the statistics: the rounding errors are independent
    and at most uniform in +-2^-4 p_j, so the RMS error is at most
    2^-4 / sqrt(3) * RMS(sqrt(sum_j p_j^2 v_j^2) / sum_j p_j) plus the bf16
    rounding; the test allows 1.5 times that. This is the bar with teeth: a
    dropped or misplaced key moves O by about |v| / n, well above it for the
    key counts used here.
LSE does not see the rounding of P, but it sees the scores' own rounding:
the FP8 MFMA does not return the exact fp32 sum of its products (measured:
score errors of about 5e-5 relative, both signs, on logits up to 80). A sum
rounded with about 14 fraction bits over a tree of 64 terms errs by at most
2^-12 times the sum of the terms' magnitudes, so with
M = |scale| * max_j sum_d |q_d k_jd| (dequantized) the bars are
|LSE - LSE_ref| <= 1e-3 + 2^-12 M, and a relative 2^-11 M on the
probabilities, i.e. one more 2^-11 M A in the elementwise bar of O.
"""
import numpy as np
import pytest

from oracle import attention
from oracle.fp8 import attention_fp8, e4m3_decode
from workloads import make_fp8

torch = pytest.importorskip("torch")
ta = pytest.importorskip("tiled_attention_16_amd")

pytestmark = pytest.mark.gpu


def dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).to("cuda")


def bf16_to_f64(t):
    return t.float().cpu().numpy().astype(np.float64)


def run_gpu(x, scale, causal, stride=None, pad_code=0):
    B, H, N_q, d = x.q8.shape
    N_k = x.k8.shape[2]
    S = stride or ta.fp8_vt_stride(N_k)
    vt = np.full((B, H, d, S), pad_code, dtype=np.uint8)
    vt[..., :N_k] = x.vt8
    o, lse = ta.attn_fwd_fp8(dev(x.q8), dev(x.k8), dev(vt), q_descale=x.q_descale, k_descale=x.k_descale,
                             v_descale=x.v_descale, causal=causal, scale=scale)
    torch.cuda.synchronize()
    return bf16_to_f64(o), lse.cpu().numpy().astype(np.float64)


def bars(x, scale, causal, rows=None):
    """Reference O, LSE and the two error bars, from the oracle's probabilities."""
    q = e4m3_decode(x.q8) * x.q_descale
    k = e4m3_decode(x.k8) * x.k_descale
    v = np.swapaxes(e4m3_decode(x.vt8), -1, -2) * x.v_descale
    o_ref, lse_ref, p = attention(q, k, v, scale, causal, rows=rows, return_probs=True)
    a = p @ np.abs(v)                # sum_j p_j |v_j| (p sums to 1)
    t = np.sqrt((p * p) @ (v * v))   # sqrt(sum_j p_j^2 v_j^2)
    n = (p > 0).sum(axis=-1, keepdims=True)
    vmax = np.abs(v).max() if v.size else 0.0
    qa = np.abs(q if rows is None else q[:, :, rows])
    mag = abs(scale) * (qa @ np.swapaxes(np.abs(k), -1, -2)).max(axis=-1, initial=0.0)   # M per row
    elem = (2.0 ** -4 + 2.0 ** -11 * mag[..., None]) * a + 2.0 ** -18 * n * vmax + 2.0 ** -8 * np.abs(o_ref) + \
        1e-6 * (a + 1e-30)
    rms = 1.5 * (2.0 ** -4 / np.sqrt(3) * np.sqrt(np.mean(t ** 2)) + 2.0 ** -8 / np.sqrt(3) *
                 np.sqrt(np.mean(o_ref ** 2))) + 1e-9
    return o_ref, lse_ref, elem, rms, mag, t


def check(o, lse, x, scale, causal, rows=None):
    o_ref, lse_ref, elem, rms, mag, _ = bars(x, scale, causal, rows)
    if rows is not None:
        o, lse = o[:, :, rows], lse[:, :, rows]
    assert np.isfinite(o).all()
    err = np.abs(o - o_ref)
    worst = np.unravel_index(np.argmax(err - elem), err.shape)
    assert np.all(err <= elem), f"elementwise bar broken at {worst}: {err[worst]} > {elem[worst]}"
    got_rms = float(np.sqrt(np.mean(err ** 2))) if err.size else 0.0
    assert got_rms <= rms, f"RMS error {got_rms} above the rounding model's {rms}"
    dead = np.isneginf(lse_ref)
    np.testing.assert_array_equal(np.isneginf(lse), dead)
    assert np.all(o[np.broadcast_to(dead[..., None], o.shape)] == 0)
    lerr = np.abs(lse[~dead] - lse_ref[~dead])
    lbar = (1e-3 + 2.0 ** -12 * mag)[~dead]
    assert np.all(lerr <= lbar), f"LSE error {lerr.max()} above its bar (largest ratio {(lerr / lbar).max():.3f})"


CASES = [
    # B, H, N_q, N_k, d, causal, seed
    (1, 2, 300, 333, 128, 0, 1),
    (2, 2, 257, 190, 64, 1, 2),
    (1, 3, 200, 260, 128, 2, 3),
    (1, 2, 130, 17, 64, 0, 4),       # fewer keys than one step
    (1, 1, 150, 100, 64, 2, 5),      # bottom-right with N_q > N_k: the first 50 rows see nothing
    (1, 2, 64, 1, 128, 1, 6),
    (2, 1, 129, 128, 128, 1, 7),     # 129 rows in one 256-row workgroup: wave 4 holds one row, waves 5-7 none
    (1, 2, 520, 520, 128, 1, 8),     # causal d=128 over three 256-row workgroups (the last of 8 rows)
    (1, 2, 600, 400, 128, 2, 9),     # bottom-right causal d=128, three workgroups, 200 rows see nothing
]


@pytest.mark.parametrize("case", CASES, ids=[f"{c[0]}x{c[1]}x{c[2]}x{c[3]}d{c[4]}c{c[5]}" for c in CASES])
def test_fp8_parity(case):
    B, H, N_q, N_k, d, causal, seed = case
    x = make_fp8(B, H, N_q, N_k, d, seed=seed, sigma=(1.0, 1.0, 1.0))
    scale = d ** -0.5
    print(f"fp8 parity {case}", flush=True)
    o, lse = run_gpu(x, scale, causal)
    check(o, lse, x, scale, causal)


def test_fp8_peaked_scores():
    """Large logits: most rows have one dominant key, P spans many binades."""
    x = make_fp8(1, 2, 200, 300, 128, seed=11, sigma=(3.0, 3.0, 1.0))
    o, lse = run_gpu(x, 0.3, 1)
    check(o, lse, x, 0.3, 1)


def test_fp8_negative_and_zero_scale():
    x = make_fp8(1, 2, 100, 150, 64, seed=12)
    for scale in (-0.125, 0.0):
        o, lse = run_gpu(x, scale, 0)
        check(o, lse, x, scale, 0)


def test_fp8_padding_is_ignored():
    """NaN codes in the row padding of V^T must not reach the output."""
    x = make_fp8(1, 2, 70, 37, 128, seed=13)
    o, lse = run_gpu(x, 128 ** -0.5, 0, stride=64, pad_code=0x7F)
    check(o, lse, x, 128 ** -0.5, 0)


def test_fp8_no_keys():
    x = make_fp8(1, 2, 40, 0, 64, seed=14)
    o, lse = run_gpu(x, 0.125, 0)
    assert np.all(o == 0) and np.all(np.isneginf(lse))


def test_fp8_matches_oracle_function():
    """The bars' own reference is the oracle's attention_fp8."""
    x = make_fp8(1, 1, 50, 70, 64, seed=15)
    o_ref, lse_ref, *_ = bars(x, 0.125, 1)
    o2, l2 = attention_fp8(x.q8, x.k8, x.vt8, 0.125, x.q_descale, x.k_descale, x.v_descale, 1)
    np.testing.assert_allclose(o_ref, o2, rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(lse_ref, l2, rtol=1e-12)


def check_whole(o, lse, x, scale, causal, row_block=1024):
    """check() over every element of a large output: per (b, h) and row
    block for the elementwise and LSE bars (the oracle's probabilities of one
    block at a time), the RMS bar over all elements together."""
    from workloads import Fp8Inputs
    B, H, N_q, _ = x.q8.shape
    err2 = t2 = o2 = 0.0
    count = 0
    for b in range(B):
        for h in range(H):
            xs = Fp8Inputs(q8=x.q8[b:b + 1, h:h + 1], k8=x.k8[b:b + 1, h:h + 1], vt8=x.vt8[b:b + 1, h:h + 1],
                           q_descale=x.q_descale, k_descale=x.k_descale, v_descale=x.v_descale)
            for r0 in range(0, N_q, row_block):
                rows = np.arange(r0, min(r0 + row_block, N_q))
                o_ref, lse_ref, elem, _, mag, t = bars(xs, scale, causal, rows)
                ob, lb = o[b:b + 1, h:h + 1, rows], lse[b:b + 1, h:h + 1, rows]
                assert np.isfinite(ob).all()
                err = np.abs(ob - o_ref)
                worst = np.unravel_index(np.argmax(err - elem), err.shape)
                assert np.all(err <= elem), f"(b, h) = ({b}, {h}) rows {r0}+: {err[worst]} > {elem[worst]}"
                dead = np.isneginf(lse_ref)
                np.testing.assert_array_equal(np.isneginf(lb), dead)
                lerr = np.abs(lb[~dead] - lse_ref[~dead])
                assert np.all(lerr <= (1e-3 + 2.0 ** -12 * mag)[~dead])
                # the RMS model's two terms, summed over every element
                t2 += float(np.sum(t ** 2))
                o2 += float(np.sum(o_ref ** 2))
                err2 += float(np.sum(err ** 2))
                count += err.size
    rms_bar = 1.5 * (2.0 ** -4 / np.sqrt(3) * np.sqrt(t2 / count) + 2.0 ** -8 / np.sqrt(3) * np.sqrt(o2 / count)) + 1e-9
    got = np.sqrt(err2 / count)
    print(f"   fp8 whole output: RMS error {got:.3e}, bar {rms_bar:.3e}", flush=True)
    assert got <= rms_bar


@pytest.mark.parametrize("B,H,N,d,causal", [(1, 32, 4096, 128, 1), (1, 16, 2048, 64, 0)])
def test_fp8_full_size_every_element(B, H, N, d, causal):
    """The benchmark's launch (and a non-causal d = 64 one), every element of O and LSE."""
    x = make_fp8(B, H, N, N, d, seed=21 if d == 128 else 23)
    print(f"fp8 whole {(B, H, N, d, causal)}", flush=True)
    o, lse = run_gpu(x, d ** -0.5, causal)
    check_whole(o, lse, x, d ** -0.5, causal)


def test_fp8_full_size_sampled_rows():
    """B=1, H=32, N=4096, d=128 causal, the benchmark's launch; sampled rows."""
    x = make_fp8(1, 32, 4096, 4096, 128, seed=21)
    o, lse = run_gpu(x, 128 ** -0.5, 1)
    rows = [0, 1, 127, 128, 255, 256, 511, 512, 1000, 2047, 2048, 3333, 4095]
    check(o, lse, x, 128 ** -0.5, 1, rows=rows)


@pytest.mark.parametrize("B,H,N,d,causal", [(1, 8, 16384, 128, 1), (1, 32, 4096, 64, 0), (2, 4, 3000, 128, 2)])
def test_fp8_large_sampled_rows(B, H, N, d, causal):
    """Long sequences and the other head dim at full size; sampled rows."""
    x = make_fp8(B, H, N, N, d, seed=22 + d)
    print(f"fp8 large {(B, H, N, d, causal)}", flush=True)
    o, lse = run_gpu(x, d ** -0.5, causal)
    rows = sorted({0, 1, 127, 128, 255, 256, 511, 512, N // 2, N - 257, N - 256, N - 129, N - 1})
    check(o, lse, x, d ** -0.5, causal, rows=rows)
