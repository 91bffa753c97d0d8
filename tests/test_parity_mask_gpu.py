"""Parity of attn_fwd_masked (a boolean mask intersected with the rules) with
the fp64 oracle, and of attn_mask_pack with a bit-by-bit reference (needs the GPU)."""
import numpy as np
import pytest

from oracle import attention, bf16_bits_to_f64, check
from workloads import WORKLOADS, make_inputs, make_random

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import tiled_attention_16_amd as ta
    ta.load_library()
    return ta


def to_dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)


def f64(t):
    return bf16_bits_to_f64(t.view(torch.int16).cpu().numpy().view(np.uint16))


def run(q, k, v, scale, causal, mask, seqlens=None, qstart=None):
    import tiled_attention_16_amd as ta
    print(f"  masked fwd B,H,Nq,Nk,d={q.shape[0]},{q.shape[1]},{q.shape[2]},{k.shape[2]},{q.shape[3]} causal={causal} "
          f"mask={mask.shape}", flush=True)
    sl = torch.from_numpy(np.asarray(seqlens, np.int32)).cuda() if seqlens is not None else None
    qs = torch.from_numpy(np.asarray(qstart, np.int32)).cuda() if qstart is not None else None
    o, lse = ta.attn_fwd(to_dev(q), to_dev(k), to_dev(v), causal=causal, scale=float(scale), seqlens_k=sl,
                         q_start=qs, attn_mask=torch.from_numpy(mask).cuda())
    torch.cuda.synchronize()
    return f64(o), lse.cpu().numpy().astype(np.float64)


def compare(q, k, v, scale, causal, mask, seqlens=None, qstart=None):
    o, lse = run(q, k, v, scale, causal, mask, seqlens, qstart)
    ro, rl = attention(bf16_bits_to_f64(q), bf16_bits_to_f64(k), bf16_bits_to_f64(v), float(scale), causal,
                       seqlens_k=seqlens, q_start=qstart, attn_mask=mask)
    r = check(o, ro, lse, rl)
    print("  ", r, flush=True)
    assert r.ok, str(r)
    return o, lse


def test_pack_matches_bit_reference():
    import tiled_attention_16_amd as ta
    rng = np.random.default_rng(3)
    m = rng.random((2, 3, 37, 300)) < 0.4
    bits, sb, sh, rw = ta.pack_mask(torch.from_numpy(m).cuda())
    torch.cuda.synchronize()
    got = bits.cpu().numpy().view(np.uint32)
    assert rw == 16 and sb == 3 * 37 * 16 and sh == 37 * 16
    want = np.zeros((2, 3, 37, rw), np.uint32)
    for j in range(300):
        want[..., j // 32] |= m[..., j].astype(np.uint32) << np.uint32(j % 32)
    np.testing.assert_array_equal(got, want)


CASES = [
    # B, H, N_q, N_k, d, causal, mask shape (b, h), density, seqlens, q_start
    (1, 2, 300, 500, 128, 0, (1, 2), 0.5, None, None),
    (2, 2, 200, 777, 64, 0, (2, 1), 0.9, None, None),
    (1, 2, 257, 257, 128, 1, (1, 1), 0.3, None, None),
    (2, 1, 300, 600, 64, 2, (2, 1), 0.6, [600, 410], [0, 20]),
    (1, 1, 64, 2100, 128, 0, (1, 1), 0.05, None, None),      # sparse: many rows see few keys
]


@pytest.mark.parametrize("case", CASES, ids=[f"{c[2]}x{c[3]}_d{c[4]}_c{c[5]}_p{c[7]}" for c in CASES])
def test_random_masks(case):
    B, H, nq, nk, d, causal, (mb, mh), dens, sl, qs = case
    q, k, v = make_random(B, H, nq, nk, d, seed=nq + nk + d)
    rng = np.random.default_rng(nq * 3 + nk)
    mask = rng.random((mb, mh, nq, nk)) < dens
    mask[0, 0, 5] = False                       # a row that sees no key
    o, lse = compare(q, k, v, np.float32(d ** -0.5), causal, mask,
                     None if sl is None else np.array(sl, np.int32), None if qs is None else np.array(qs, np.int32))
    assert np.all(o[0, 0, 5] == 0) and np.isneginf(lse[0, 0, 5])


def test_mask_equal_to_the_causal_rule_gives_the_same_bits():
    import tiled_attention_16_amd as ta
    q, k, v = make_random(1, 2, 700, 700, 128, seed=91)
    tq, tk, tv = to_dev(q), to_dev(k), to_dev(v)
    tril = torch.tril(torch.ones(700, 700, dtype=torch.bool, device="cuda"))[None, None]
    o1, l1 = ta.attn_fwd(tq, tk, tv, causal=True)
    o2, l2 = ta.attn_fwd(tq, tk, tv, attn_mask=tril)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(l1, l2)


def test_sliding_window_full_size():
    """The causal N = 4096 workload with a 1024-key sliding window (key j visible
    to row i iff i - 1024 < j <= i) as a mask shared by all heads; sampled rows."""
    import tiled_attention_16_amd as ta
    w = WORKLOADS["causal_n4096_d128"]
    inp = make_inputs(w)
    i = np.arange(w.N_q)[:, None]
    j = np.arange(w.N_k)[None, :]
    mask = ((j > i - 1024) & (j <= i))[None, None]
    o, lse = ta.attn_fwd(to_dev(inp.q), to_dev(inp.k), to_dev(inp.v), causal=True, scale=float(inp.scale),
                         attn_mask=torch.from_numpy(mask).cuda())
    torch.cuda.synchronize()
    o, lse = f64(o), lse.cpu().numpy().astype(np.float64)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))
    rng = np.random.default_rng(5)
    rows = np.unique(np.concatenate([[0, 1, 1023, 1024, 1025, 2047, 4095], rng.choice(w.N_q, 40, replace=False)]))
    for b, h in [(0, 0), (0, 31)]:
        ro, rl = attention(bf16_bits_to_f64(inp.q[b:b + 1, h:h + 1]), bf16_bits_to_f64(inp.k[b:b + 1, h:h + 1]),
                           bf16_bits_to_f64(inp.v[b:b + 1, h:h + 1]), float(inp.scale), True, rows=rows,
                           attn_mask=mask)
        r = check(o[b:b + 1, h:h + 1, rows], ro, lse[b:b + 1, h:h + 1, rows], rl)
        print(f"  window b={b} h={h}: {r}", flush=True)
        assert r.ok, str(r)


@pytest.mark.parametrize("d", [64, 128])
def test_first_allowed_key_late_with_large_logits(d):
    """Rows whose first allowed key comes slices after key 0 (the mask hides
    their first 40..300 keys), with logits large enough that the running
    maximum must be set and raised late: both O and the LSE must match."""
    B, H, n = 1, 2, 400
    q, k, v = make_random(B, H, n, n, d, seed=97 + d, sigma=(4.0, 1.0, 1.0))
    rng = np.random.default_rng(98)
    mask = rng.random((1, 1, n, n)) < 0.3
    first = rng.integers(40, 300, size=n)
    for i in range(n):
        if i % 2:
            mask[0, 0, i, :first[i]] = False
    compare(q, k, v, np.float32(d ** -0.5), 0, mask)


# ---------------------------------------------------------------- block-sparse (attn_fwd_block_sparse)
SPARSE = [
    # B, H, N_q, N_k, d, causal, block-mask shape (b, h), density, seqlens, q_start
    (1, 2, 300, 700, 128, 0, (1, 2), 0.5, None, None),
    (2, 1, 600, 600, 64, 1, (2, 1), 0.6, [600, 333], [0, 100]),
    (1, 1, 512, 2100, 128, 0, (1, 1), 0.2, None, None),
    (1, 2, 257, 1000, 128, 2, (1, 1), 0.7, None, None),
]


@pytest.mark.parametrize("case", SPARSE, ids=[f"{c[2]}x{c[3]}_d{c[4]}_c{c[5]}_p{c[7]}" for c in SPARSE])
def test_block_sparse(case):
    import tiled_attention_16_amd as ta
    from oracle import expand_block_mask
    B, H, nq, nk, d, causal, (mb, mh), dens, sl, qs = case
    q, k, v = make_random(B, H, nq, nk, d, seed=nq + 13 * nk + d)
    rng = np.random.default_rng(nq + 17 * nk)
    nqb, nkb = -(-nq // 256), -(-nk // 128)
    bm = rng.random((mb, mh, nqb, nkb)) < dens
    bm[0, 0, 0, :] = False                    # a tile with no block at all: its rows output 0
    scale = np.float32(d ** -0.5)
    slt = torch.from_numpy(np.array(sl, np.int32)).cuda() if sl is not None else None
    qst = torch.from_numpy(np.array(qs, np.int32)).cuda() if qs is not None else None
    print(f"  block-sparse {case}", flush=True)
    o, lse = ta.attn_fwd(to_dev(q), to_dev(k), to_dev(v), causal=causal, scale=float(scale), seqlens_k=slt,
                         q_start=qst, block_mask=torch.from_numpy(bm).cuda())
    torch.cuda.synchronize()
    o, lse = f64(o), lse.cpu().numpy().astype(np.float64)
    ro, rl = attention(bf16_bits_to_f64(q), bf16_bits_to_f64(k), bf16_bits_to_f64(v), float(scale), causal,
                       seqlens_k=None if sl is None else np.array(sl), q_start=None if qs is None else np.array(qs),
                       attn_mask=expand_block_mask(bm, nq, nk, 256, 128))
    r = check(o, ro, lse, rl)
    print("  ", r, flush=True)
    assert r.ok, str(r)
    assert np.all(o[0, 0, :256] == 0) and np.all(np.isneginf(lse[0, 0, :256]))


def test_block_sparse_all_kept_equals_plain():
    import tiled_attention_16_amd as ta
    q, k, v = make_random(1, 2, 700, 700, 128, seed=111)
    tq, tk, tv = to_dev(q), to_dev(k), to_dev(v)
    bm = torch.ones((1, 1, 3, 6), dtype=torch.bool, device="cuda")
    o1, l1 = ta.attn_fwd(tq, tk, tv, causal=True)
    o2, l2 = ta.attn_fwd(tq, tk, tv, causal=True, block_mask=bm)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)) and torch.equal(l1, l2)


def test_block_sparse_full_size_sampled():
    """The causal N = 4096 workload with half of its blocks kept (one mask for all heads)."""
    import tiled_attention_16_amd as ta
    from oracle import expand_block_mask
    w = WORKLOADS["causal_n4096_d128"]
    inp = make_inputs(w)
    bm = np.random.default_rng(7).random((1, 1, 16, 32)) < 0.5
    o, lse = ta.attn_fwd(to_dev(inp.q), to_dev(inp.k), to_dev(inp.v), causal=True, scale=float(inp.scale),
                         block_mask=torch.from_numpy(bm).cuda())
    torch.cuda.synchronize()
    o, lse = f64(o), lse.cpu().numpy().astype(np.float64)
    rows = np.unique(np.concatenate([[0, 255, 256, 2047, 4095], np.random.default_rng(8).choice(4096, 40, replace=False)]))
    full = expand_block_mask(bm, 4096, 4096, 256, 128)
    for b, h in [(0, 0), (0, 31)]:
        ro, rl = attention(bf16_bits_to_f64(inp.q[b:b + 1, h:h + 1]), bf16_bits_to_f64(inp.k[b:b + 1, h:h + 1]),
                           bf16_bits_to_f64(inp.v[b:b + 1, h:h + 1]), float(inp.scale), True, rows=rows, attn_mask=full)
        r = check(o[b:b + 1, h:h + 1, rows], ro, lse[b:b + 1, h:h + 1, rows], rl)
        print(f"  block-sparse b={b} h={h}: {r}", flush=True)
        assert r.ok, str(r)


# Run as the first launches of a fresh process (cold caches and address
# translations, freshly allocated inputs): the boolean-mask d = 64 shapes whose
# first tiles, in a build that awaited only the oldest of a tile's first copies
# before its first barrier, read stale K/V or mask words on such launches.
_FIRST_LAUNCH = r'''
import sys
import numpy as np
import torch
import tiled_attention_16_amd as ta
from oracle import attention, bf16_bits_to_f64, check
from workloads import make_random

def to_dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)

ok = True
for case in range(2):
    if case == 0:
        B, H, n_q, n_k, d = 2, 2, 200, 777, 64
        q, k, v = make_random(B, H, n_q, n_k, d, seed=n_q + n_k + d)
        mask = np.random.default_rng(n_q * 3 + n_k).random((2, 1, n_q, n_k)) < 0.9
        mask[0, 0, 5] = False
    else:
        B, H, n_q, n_k, d = 1, 2, 400, 400, 64
        q, k, v = make_random(B, H, n_q, n_k, d, seed=97 + d, sigma=(4.0, 1.0, 1.0))
        rng = np.random.default_rng(98)
        mask = rng.random((1, 1, n_q, n_k)) < 0.3
        first = rng.integers(40, 300, size=n_q)
        for i in range(1, n_q, 2):
            mask[0, 0, i, :first[i]] = False
    o, lse = ta.attn_fwd(to_dev(q), to_dev(k), to_dev(v), causal=0, scale=float(d ** -0.5),
                         attn_mask=torch.from_numpy(mask).cuda())
    torch.cuda.synchronize()
    o = bf16_bits_to_f64(o.view(torch.int16).cpu().numpy().view(np.uint16))
    ro, rl = attention(bf16_bits_to_f64(q), bf16_bits_to_f64(k), bf16_bits_to_f64(v), d ** -0.5, 0, attn_mask=mask)
    r = check(o, ro, lse.cpu().numpy().astype(np.float64), rl)
    print(f"case {case}: {r}", flush=True)
    ok = ok and r.ok
print("OK" if ok else "FAIL", flush=True)
sys.exit(0 if ok else 1)
'''


def test_first_launch_in_a_fresh_process():
    import os
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    env = dict(os.environ, PYTHONPATH=root + os.pathsep + os.environ.get("PYTHONPATH", ""))
    r = subprocess.run([sys.executable, "-u", "-c", _FIRST_LAUNCH], cwd=root, env=env, capture_output=True,
                       text=True, timeout=240)
    print(r.stdout, flush=True)
    assert r.returncode == 0 and "OK" in r.stdout, r.stdout + r.stderr[-2000:]
